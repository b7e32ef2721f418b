"""GPU parity: every C-ABI call against the CPU oracle on the same seeded inputs.

Bar: packed bytes, codes, code sums and int32 accumulators bit-exact; float32
scales and outputs within 1e-5 relative (outputs with acc == 0 exactly 0); on
the Hadamard path at most 0.01% of codes may differ, by one, at rounding ties.
Full-size workloads (the benchmark's shapes and launch configuration) are
checked on sampled outputs the oracle computes one by one.
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
    err = np.abs(got - want)
    bad = err > rtol * np.abs(want)
    assert not bad.any(), (f"{bad.sum()} of {bad.size} values off by more than {rtol} relative; "
                           f"first at {np.argwhere(bad)[0]}: got {got[bad][0]} want {want[bad][0]}")


# ---------------------------------------------------------------------------
# Weight quantisation and packing.
# ---------------------------------------------------------------------------

PACK_CASES = [
    (512, 256, False),       # tiny BitLinear
    (4096, 4096, False),     # decode q/o projection
    (11008, 4096, False),    # decode up projection (N = 11008)
    (4096, 11008, False),    # decode down projection (K = 11008)
    (1, 64, False),          # smallest
    (37, 192, False),        # ragged rows, K not a power of two
    (70, 128, False),        # two row blocks, the second ragged; two K stages
    (300, 4096, True),       # H-BitLinear weights
    (4096, 16384, True),     # H-BitLinear down projection
    (33, 256, True),
    (5, 32768, True),        # largest Hadamard
]


@pytest.mark.parametrize("N,K,hadamard", PACK_CASES)
def test_pack_weights(orc, dev, N, K, hadamard):
    W = synth.weights(N, K, seed=100 + N % 97 + K % 89)
    want_packed, want_dw, want_sw, _ = orc.pack_weights(W, hadamard=hadamard)
    packed, w_scale = bt.pack_weights(to_dev(W, dev), hadamard=hadamard)
    got = host(packed)
    mism = np.count_nonzero(got != want_packed)
    assert mism == 0, f"{mism} packed bytes differ"
    ws = host(w_scale)
    assert ws[1] == want_sw, (ws[1], want_sw)
    assert ws[0] == want_dw, (ws[0], want_dw)


def test_pack_all_zero_and_ternary_inputs(orc, dev):
    packed, w_scale = bt.pack_weights(torch.zeros((9, 128), dtype=torch.float32, device=dev))
    assert (host(packed) == 0x55).all() and (host(w_scale) == 0).all()
    q = np.random.default_rng(7).integers(-1, 2, size=(64, 256)).astype(np.float32)
    want, _, _, _ = orc.pack_weights(q)
    got, _ = bt.pack_weights(to_dev(q, dev))
    np.testing.assert_array_equal(host(got), want)


# ---------------------------------------------------------------------------
# Activation quantisation (int8) and Hadamard + int4.
# ---------------------------------------------------------------------------

def _activation(M, K, seed, dist="normal", frac=0.01, factor=20.0):
    return synth.activations(M, K, seed, seed + 1, dist=dist, outlier_frac=frac, outlier_factor=factor)


QUANT_CASES = [
    (4, 256, False), (1, 4096, False), (1, 11008, False), (3, 14336, True), (2048, 4096, False),
    (17, 65536, True), (5, 64, False), (33, 192, True),
    (3, 32768, False), (2, 20480, True), (6, 16384, True), (4, 16448, False),   # 256 / 1024 threads
]


@pytest.mark.parametrize("M,K,with_gain", QUANT_CASES)
def test_quant_act(orc, dev, M, K, with_gain):
    x = _activation(M, K, seed=200 + K % 101, frac=0.005, factor=50.0)
    gain = (np.random.default_rng(K).uniform(0.5, 1.5, K).astype(np.float32) if with_gain else None)
    wq, wdx, wqs = orc.quant_act(x, gain=gain, eps=1e-5)
    q, dx, qs = bt.quant_act(bf16_to_dev(x, dev), None if gain is None else to_dev(gain, dev), 1e-5)
    np.testing.assert_array_equal(host(q), wq)
    np.testing.assert_array_equal(host(qs), wqs)
    assert_close_rel(host(dx), wdx)


def test_quant_act_zero_tiny_and_tie_tokens(orc, dev):
    x = np.zeros((4, 256), np.float32)
    x[1, 3] = 2.0 ** -126
    x[2, :5] = [127.0, 2.5, 3.5, -2.5, -3.5]
    x[3] = np.linspace(-3, 3, 256)
    bits = synth.bf16_bits(x)
    wq, wdx, wqs = orc.quant_act(bits)
    q, dx, qs = bt.quant_act(bf16_to_dev(bits, dev))
    np.testing.assert_array_equal(host(q), wq)
    np.testing.assert_array_equal(host(qs), wqs)
    assert_close_rel(host(dx), wdx)
    assert host(dx)[0] == 0 and host(dx)[1] == 0


HQ_CASES = [
    (4, 256, False), (3, 512, True), (5, 1024, False), (7, 2048, True), (512, 4096, False),
    (2, 8192, True), (512, 16384, False), (3, 32768, True),
]


@pytest.mark.parametrize("M,K,with_gain", HQ_CASES)
def test_hadamard_quant_act(orc, dev, M, K, with_gain):
    x = _activation(M, K, seed=300 + K % 103, dist="student_t", frac=0.0)
    gain = (np.random.default_rng(K + 1).uniform(0.5, 1.5, K).astype(np.float32) if with_gain else None)
    wq, wdx, wqs = orc.hadamard_quant_act(x, gain=gain, eps=1e-5)
    q, dx, qs = bt.hadamard_quant_act(bf16_to_dev(x, dev), None if gain is None else to_dev(gain, dev))
    q = host(q)
    diff = np.abs(q.astype(np.int16) - wq.astype(np.int16))
    assert diff.max() <= 1
    assert np.count_nonzero(diff) <= 1e-4 * q.size
    assert np.count_nonzero(diff) == 0, "same stage order should give identical codes"
    np.testing.assert_array_equal(host(qs), wqs)
    assert_close_rel(host(dx), wdx)


# ---------------------------------------------------------------------------
# Contraction + dequantisation.
# ---------------------------------------------------------------------------

def _forward_inputs(orc, M, N, K, seed, hadamard=False):
    W = synth.weights(N, K, seed)
    packed, d_w, _, _ = orc.pack_weights(W, hadamard=hadamard)
    x = _activation(M, K, seed + 7, dist="student_t" if hadamard else "normal")
    quant = orc.hadamard_quant_act if hadamard else orc.quant_act
    xq, d_x, qsum = quant(x)
    return packed, np.array([d_w, 0], np.float32), xq, d_x, qsum


def _run_forward(dev, packed, w_scale, xq, d_x, qsum):
    y, acc = bt.linear_forward(to_dev(xq, dev), to_dev(d_x, dev), to_dev(qsum, dev),
                               to_dev(packed, dev), to_dev(w_scale, dev), return_acc=True)
    return host(y), host(acc)


FORWARD_FULL_CASES = [
    # GEMV (M <= 4)
    (1, 512, 256), (1, 4096, 4096), (1, 11008, 4096), (1, 4096, 11008), (2, 1000, 4096),
    (3, 77, 14336), (4, 4097, 8192), (1, 1, 64), (1, 130, 32768), (2, 9, 16384),
    (1, 40000, 4096),    # 10 rows per wave in 4096 waves
    (1, 70000, 4096),    # 35 rows per wave: two alternating register sets
    (2, 6000, 12288),    # 2 tokens x 3 chunks per lane: alternating one-row sets
    (1, 8192, 28672),    # 7 chunks (run as 8), 4 rows per wave: alternating one-row sets
    # matrix-core GEMM
    (5, 512, 256), (16, 4096, 4096), (17, 1000, 4096), (64, 1024, 4096), (100, 333, 192),
    (128, 128, 128), (256, 1024, 4096), (300, 4099, 1024), (1, 70, 65536), (33, 65, 64),
    # each matrix-core tile size at ragged M, N and K (K not a multiple of the 256-deep stage)
    (2100, 14000, 192),  # 448 x 128 tiles, two or more rounds
    (900, 14000, 192),   # 448 x 128 tiles, one round
    (2000, 4100, 64),    # 128 x 128 tiles
    (999, 4100, 320),    # 128 x 128 tiles, about one round
    (250, 16400, 192),   # 128 x 128 tiles (few tokens, many rows)
    (300, 5000, 320),    # 128 x 64 tiles in two K groups
    (300, 4000, 320),    # 64 x 64 tiles in two K groups
    (200, 900, 4160),    # 64 x 64 tiles in four K groups (17 stages: three groups run past K)
    (100, 333, 12352),   # 64 x 64 tiles in four K groups (49 stages)
    (9, 4100, 576),      # skinny, one row block per workgroup, K split over eight waves
    (16, 9000, 1088),    # skinny, two row blocks
    (7, 6000, 4096),     # skinny, two row blocks, ragged N
    (12, 12300, 320),    # skinny, four row blocks, K split over eight waves
    (16, 30000, 192),    # skinny, four row blocks, K split over four waves
]


@pytest.mark.parametrize("M,N,K", FORWARD_FULL_CASES)
def test_linear_forward(orc, dev, M, N, K):
    packed, w_scale, xq, d_x, qsum = _forward_inputs(orc, M, N, K, seed=400 + M + N % 113)
    y, acc = _run_forward(dev, packed, w_scale, xq, d_x, qsum)
    want_acc, want_y = orc.linear_forward(xq, d_x, packed, w_scale[0], K)
    mism = np.count_nonzero(acc != want_acc)
    assert mism == 0, f"{mism} of {acc.size} accumulators differ; first {np.argwhere(acc != want_acc)[0]}"
    assert_close_rel(y, want_y)
    assert (y[want_acc == 0] == 0).all()


FORWARD_SAMPLED_CASES = [
    (2048, 14336, 4096, False),   # prefill FFN up projection
    (2048, 4096, 4096, False),    # prefill attention projection
    (1024, 4096, 4096, False),
    (512, 4096, 4096, True),      # H-BitLinear
    (512, 4096, 16384, True),     # H-BitLinear down projection
    (256, 14336, 4096, False),    # Llama-3-8B block gate/up at M = 256
    (16, 14336, 4096, False),     # ... at M = 16
    (256, 4096, 14336, False),    # down projection at M = 256
    (256, 28672, 4096, False),    # grouped gate|up at M = 256 (128 x 128 tiles)
    (1000, 2100, 12352, False),   # 128 x 64 tiles in three K groups, ragged M, N and K
]


@pytest.mark.parametrize("M,N,K,hadamard", FORWARD_SAMPLED_CASES)
def test_linear_forward_full_size_sampled(orc, dev, M, N, K, hadamard):
    packed, w_scale, xq, d_x, qsum = _forward_inputs(orc, M, N, K, seed=500 + M, hadamard=hadamard)
    y, acc = _run_forward(dev, packed, w_scale, xq, d_x, qsum)
    rng = np.random.default_rng(M + N + K)
    rows = np.concatenate([rng.integers(0, M, 3000), np.full(N, M - 1), np.zeros(64, np.int64)])
    cols = np.concatenate([rng.integers(0, N, 3000), np.arange(N), np.arange(N - 64, N)])
    want = orc.int_gemm_sampled(xq, packed, K, rows, cols)
    got = acc[rows, cols]
    assert np.count_nonzero(got != want) == 0
    want_y = want.astype(np.float64) * d_x[rows].astype(np.float64) * np.float64(w_scale[0])
    assert_close_rel(y[rows, cols], want_y)
    # properties at every output: y is the dequantised accumulator
    assert_close_rel(y, acc.astype(np.float64) * d_x[:, None].astype(np.float64) * np.float64(w_scale[0]))


def test_forward_determinism(orc, dev):
    packed, w_scale, xq, d_x, qsum = _forward_inputs(orc, 64, 4096, 4096, seed=600)
    args = [to_dev(a, dev) for a in (xq, d_x, qsum, packed, w_scale)]
    first = None
    for _ in range(5):
        y, acc = bt.linear_forward(*args, return_acc=True)
        cur = (host(y), host(acc))
        if first is None:
            first = cur
        else:
            np.testing.assert_array_equal(cur[1], first[1])
            np.testing.assert_array_equal(cur[0], first[0])


def test_empty_inputs(dev):
    xq = torch.empty((0, 256), dtype=torch.int8, device=dev)
    packed = torch.full((8, 64), 0x55, dtype=torch.uint8, device=dev)
    ws = torch.ones(2, dtype=torch.float32, device=dev)
    y = bt.linear_forward(xq, torch.empty(0, device=dev), torch.empty(0, dtype=torch.int32, device=dev),
                          packed, ws)
    assert tuple(y.shape) == (0, 8)
    q, dx, qs = bt.quant_act(torch.empty((0, 128), dtype=torch.bfloat16, device=dev))
    assert q.shape[0] == 0 and dx.shape[0] == 0
    xq = torch.ones((3, 256), dtype=torch.int8, device=dev)
    y = bt.linear_forward(xq, torch.ones(3, device=dev), torch.zeros(3, dtype=torch.int32, device=dev),
                          torch.empty((0, 64), dtype=torch.uint8, device=dev), ws)
    assert tuple(y.shape) == (3, 0)
    # packed 4-bit codes and the warm-up blend
    q4, dx4, qs4 = bt.hadamard_quant_act_i4(torch.empty((0, 256), dtype=torch.bfloat16, device=dev))
    assert tuple(q4.shape) == (0, 128) and dx4.shape[0] == 0 and qs4.shape[0] == 0
    y = bt.linear_forward_i4(q4, dx4, qs4, packed, ws)
    assert tuple(y.shape) == (0, 8)
    y = bt.linear_forward_i4(torch.zeros((2, 128), dtype=torch.uint8, device=dev), torch.ones(2, device=dev),
                             torch.zeros(2, dtype=torch.int32, device=dev),
                             torch.empty((0, 64), dtype=torch.uint8, device=dev), ws)
    assert tuple(y.shape) == (2, 0)
    W = torch.zeros((8, 256), dtype=torch.float32, device=dev)
    y = bt.linear_forward_blend(torch.empty((0, 256), dtype=torch.bfloat16, device=dev), W, packed, ws, 0.5)
    assert tuple(y.shape) == (0, 8)


# ---------------------------------------------------------------------------
# End to end through the GPU path only, compared with the oracle end to end.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("workload", ["tiny", "decode"])
def test_bitlinear_end_to_end(orc, dev, workload):
    for layer in synth.workload(workload):
        W, x = layer.weights(), layer.activations()
        packed, d_w, _, _ = orc.pack_weights(W)
        xq, d_x, _ = orc.quant_act(x)
        want_acc, want_y = orc.linear_forward(xq, d_x, packed, d_w, layer.K)
        layer_gpu = bt.BitLinear(to_dev(W, dev))
        y = host(layer_gpu(bf16_to_dev(x, dev)))
        assert_close_rel(y, want_y)


def test_hadamard_bitlinear_end_to_end(orc, dev):
    M, N, K = 32, 256, 1024
    W = synth.weights(N, K, 700)
    x = _activation(M, K, 701, dist="student_t", frac=0.0)
    packed, d_w, _, _ = orc.pack_weights(W, hadamard=True)
    xq, d_x, _ = orc.hadamard_quant_act(x)
    _, want_y = orc.linear_forward(xq, d_x, packed, d_w, K)
    layer = bt.BitLinear(to_dev(W, dev), hadamard=True)
    assert_close_rel(host(layer(bf16_to_dev(x, dev))), want_y)


# ---------------------------------------------------------------------------
# Fused forward (quantisation inside the contraction kernel for M <= 4).
# ---------------------------------------------------------------------------

FUSED_CASES = [
    (1, 4096, 4096, False), (1, 11008, 4096, False), (1, 4096, 11008, True), (2, 1000, 4096, False),
    (3, 77, 8192, True), (4, 4097, 8192, False), (1, 33, 32768, False), (1, 1, 64, True),
    (1, 14336, 4096, False), (1, 4096, 14336, False), (4, 300, 256, True),
    (5, 100, 1024, False), (64, 257, 4096, True),     # two-kernel path (M > 4)
    (2, 50, 32768, False),                             # M * K beyond the fused limit
    # more rows per wave than one register set holds (two alternating sets):
    (1, 40000, 4096, False),                           # 1 chunk per lane, 10 rows per wave (4096 waves)
    (1, 70000, 4096, False),                           # 1 chunk, 35 rows per wave (2048 waves, two sets)
    (1, 36000, 8192, True),                            # 2 chunks, 18 rows per wave (2048 waves, two sets)
    (1, 28672, 8192, False),                           # 2 chunks, 7 rows per wave (4096 waves)
    (1, 8192, 28672, True),                            # 7 chunks (run as 8), 4 rows per wave
    (1, 20000, 16384, False),                          # 4 chunks, 10 rows per wave
    (2, 6000, 12288, False),                           # 2 tokens x 3 chunks: one-row sets
    (4, 9000, 8192, True),                             # 4 tokens x 2 chunks: one-row sets
    # one-token kernel with exact rows per wave (N < 16384, ceil(N / 1024) rows):
    (1, 16383, 4096, True),                            # 16 rows per wave, last wave ragged
    (1, 5000, 8192, False),                            # 2 chunks, 5 rows per wave
    (1, 3000, 12288, True),                            # 3 chunks, 3 rows per wave
    (1, 1025, 192, False),                             # 2 rows per wave, one chunk of three lanes
    (1, 700, 16384, True),                             # 4 chunks, one row per wave, 700 waves
    (1, 8193, 8192, False),                            # 2 chunks past one register set: decode_kernel
    (1, 28672, 4096, False),                           # Llama-3-8B gate|up: decode_kernel
    (1, 32767, 4096, True),                            # decode_kernel, last wave ragged
    (1, 20000, 8192, False),                           # 2 chunks, 20 rows per wave: decode_kernel
    (1, 12000, 8192, True),                            # 2 chunks, 12 rows per wave: decode_kernel
    (1, 9000, 14336, False),                           # 4 chunks, 9 rows per wave: decode_kernel
    (1, 8000, 14336, True),                            # 4 chunks, 8 rows per wave: decode_kernel
]


@pytest.mark.parametrize("M,N,K,with_gain", FUSED_CASES)
def test_bitlinear_forward_fused(orc, dev, M, N, K, with_gain):
    W = synth.weights(N, K, seed=800 + N % 71)
    x = _activation(M, K, seed=801 + K % 67)
    gain = np.random.default_rng(N + K).uniform(0.5, 1.5, K).astype(np.float32) if with_gain else None
    packed, d_w, _, _ = orc.pack_weights(W)
    wq, wdx, wqs = orc.quant_act(x, gain=gain)
    want_acc, want_y = orc.linear_forward(wq, wdx, packed, d_w, K)
    w_scale = np.array([d_w, 0], np.float32)
    codes = (torch.empty((M, K), dtype=torch.int8, device=dev), torch.empty(M, device=dev),
             torch.empty(M, dtype=torch.int32, device=dev))
    acc = torch.empty((M, N), dtype=torch.int32, device=dev)
    y, acc = bt.bitlinear_forward(bf16_to_dev(x, dev), to_dev(packed, dev), to_dev(w_scale, dev),
                                  None if gain is None else to_dev(gain, dev), 1e-5, codes=codes,
                                  acc_out=acc)
    np.testing.assert_array_equal(host(codes[0]), wq)
    np.testing.assert_array_equal(host(codes[2]), wqs)
    assert_close_rel(host(codes[1]), wdx)
    np.testing.assert_array_equal(host(acc), want_acc)
    assert_close_rel(host(y), want_y)


def test_bitlinear_forward_graph_replays(orc, dev):
    """The fused decode captured in a HIP graph: every replay matches the eager result."""
    M, N, K = 1, 4096, 4096
    W = synth.weights(N, K, 900)
    packed_np, d_w, _, _ = orc.pack_weights(W)
    packed, w_scale = to_dev(packed_np, dev), to_dev(np.array([d_w, 0], np.float32), dev)
    xs = [bf16_to_dev(_activation(M, K, 901 + i), dev) for i in range(3)]
    x = xs[0].clone()
    codes = (torch.empty((M, K), dtype=torch.int8, device=dev), torch.empty(M, device=dev),
             torch.empty(M, dtype=torch.int32, device=dev))
    y = torch.empty((M, N), device=dev)
    eager = []
    for xi in xs:
        eager.append(host(bt.bitlinear_forward(xi, packed, w_scale)).copy())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            bt.bitlinear_forward(x, packed, w_scale, out=y, codes=codes)
    torch.cuda.current_stream().wait_stream(side)
    for rep in range(6):
        i = rep % 3
        x.copy_(xs[i])
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(y), eager[i])


# ---------------------------------------------------------------------------
# Grouped forward: projections sharing one input, stacked row-wise, one launch.
# ---------------------------------------------------------------------------

GROUPED_CASES = [
    (1, 4096, (4096, 1024, 1024), False),     # Llama-3-8B q|k|v, decode
    (1, 4096, (14336, 14336), False),         # gate|up, decode
    (3, 256, (37, 64, 5), True),              # ragged groups, fused path
    (16, 4096, (4096, 1024, 1024), False),    # skinny path
    (256, 4096, (1024, 512, 512), False),     # tiled GEMM path
    (100, 192, (50, 77, 3, 1, 9, 33, 2, 64), True),  # eight groups, ragged
    (2100, 192, (7000, 6999, 1), False),      # 448 x 128 tiles across group borders
]


@pytest.mark.parametrize("M,K,rows,with_gain", GROUPED_CASES)
def test_bitlinear_forward_grouped(orc, dev, M, K, rows, with_gain):
    x = _activation(M, K, seed=1100 + M)
    gain = np.random.default_rng(M + K).uniform(0.5, 1.5, K).astype(np.float32) if with_gain else None
    wq, wdx, wqs = orc.quant_act(x, gain=gain)
    packs, scales, want_acc, want_y = [], [], [], []
    for g, n in enumerate(rows):
        W = synth.weights(n, K, seed=1200 + 10 * g + n % 7)
        packed, d_w, s_w, _ = orc.pack_weights(W)
        acc_g, y_g = orc.linear_forward(wq, wdx, packed, d_w, K)
        packs.append(packed)
        scales.append([d_w, s_w])
        want_acc.append(acc_g)
        want_y.append(y_g)
    N = sum(rows)
    codes = (torch.empty((M, K), dtype=torch.int8, device=dev), torch.empty(M, device=dev),
             torch.empty(M, dtype=torch.int32, device=dev))
    acc = torch.empty((M, N), dtype=torch.int32, device=dev)
    y, acc = bt.bitlinear_forward_grouped(
        bf16_to_dev(x, dev), to_dev(np.concatenate(packs), dev),
        to_dev(np.array(scales, np.float32), dev), rows,
        None if gain is None else to_dev(gain, dev), 1e-5, codes=codes, acc_out=acc)
    np.testing.assert_array_equal(host(codes[0]), wq)
    np.testing.assert_array_equal(host(codes[2]), wqs)
    np.testing.assert_array_equal(host(acc), np.concatenate(want_acc, axis=1))
    assert_close_rel(host(y), np.concatenate(want_y, axis=1))


def test_pack_weights_grouped_matches_single_packs(orc, dev):
    K, rows = 512, (96, 32, 160)
    Ws = [synth.weights(n, K, seed=1300 + g) for g, n in enumerate(rows)]
    packed, w_scales, got_rows = bt.pack_weights_grouped([to_dev(W, dev) for W in Ws])
    assert got_rows == list(rows)
    want = [orc.pack_weights(W) for W in Ws]
    np.testing.assert_array_equal(host(packed), np.concatenate([p for p, *_ in want]))
    np.testing.assert_array_equal(host(w_scales), np.array([[d, s] for _, d, s, _ in want], np.float32))


# ---------------------------------------------------------------------------
# True 4-bit H path: 6-bit E3M2 activation codes, FP4 x FP6 matrix cores.
# ---------------------------------------------------------------------------

import f6_layout  # noqa: E402  (host encoder/decoder of the xq6 layout)


@pytest.mark.parametrize("M,K,with_gain", [(1, 256, False), (7, 4096, True), (512, 4096, False),
                                            (33, 16384, False), (2, 32768, True)])
def test_hadamard_quant_act_f6(orc, dev, M, K, with_gain):
    x = _activation(M, K, seed=1400 + M, dist="student_t")
    gain = np.random.default_rng(K).uniform(0.5, 1.5, K).astype(np.float32) if with_gain else None
    wq, wdx, wqs = orc.hadamard_quant_act(x, gain=gain)
    xq6, xs, qs = bt.hadamard_quant_act_f6(bf16_to_dev(x, dev),
                                           None if gain is None else to_dev(gain, dev))
    got = f6_layout.decode(host(xq6), K)
    # the GPU keeps the transform's float order, so the codes match exactly
    np.testing.assert_array_equal(got, wq)
    np.testing.assert_array_equal(host(qs), wqs)
    assert_close_rel(host(xs), wdx)


F6_FORWARD_CASES = [
    (1, 100, 256), (3, 77, 4096), (64, 333, 1024), (200, 900, 2048), (100, 250, 320),
    (2100, 14000, 256),   # 448 x 128 tiles
    (2000, 4100, 192),    # 128 x 128 tiles, K not a multiple of the 256-deep stage
    (512, 4096, 64),      # 128 x 64 tiles in two K groups
    (300, 4000, 320),     # 64 x 64 tiles in two K groups
    (100, 333, 12352),    # 64 x 64 tiles in four K groups
]


@pytest.mark.parametrize("M,N,K", F6_FORWARD_CASES)
def test_linear_forward_f6(orc, dev, M, N, K):
    rng = np.random.default_rng(M * 7 + N + K)
    codes = rng.integers(-8, 8, (M, K)).astype(np.int8)
    codes[0, :] = 0                                   # an all-zero token
    if M > 2:
        codes[1, :] = -8                              # extreme codes
    W = synth.weights(N, K, seed=1500 + N % 97)
    packed, d_w, _, _ = orc.pack_weights(W)
    d_x = rng.uniform(1e-3, 1e-2, M).astype(np.float32)
    qsum = codes.astype(np.int64).sum(axis=1).astype(np.int32)
    want_acc, want_y = orc.linear_forward(codes, d_x, packed, d_w, K)
    y, acc = bt.linear_forward_f6(to_dev(f6_layout.encode(codes), dev), to_dev(d_x, dev),
                                  to_dev(qsum, dev), to_dev(packed, dev),
                                  to_dev(np.array([d_w, 0], np.float32), dev), return_acc=True)
    np.testing.assert_array_equal(host(acc), want_acc)
    assert_close_rel(host(y), want_y)


@pytest.mark.parametrize("K", [4096, 16384])
def test_h_bitlinear_f6_matches_int8_path(orc, dev, K):
    """Full H-BitLinear at the benchmark shapes: the f6 path gives the int8 path's
    accumulators and outputs bit for bit, and both match the oracle on samples."""
    M, N = 512, 4096
    W = synth.weights(N, K, 1600)
    x_bits = _activation(M, K, 1601, dist="student_t")
    x = bf16_to_dev(x_bits, dev)
    packed, w_scale = bt.pack_weights(to_dev(W, dev), hadamard=True)
    xq, xs, qs = bt.hadamard_quant_act(x)
    y8, acc8 = bt.linear_forward(xq, xs, qs, packed, w_scale, return_acc=True)
    xq6, xs6, qs6 = bt.hadamard_quant_act_f6(x)
    y6, acc6 = bt.linear_forward_f6(xq6, xs6, qs6, packed, w_scale, return_acc=True)
    np.testing.assert_array_equal(host(acc6), host(acc8))
    np.testing.assert_array_equal(host(y6), host(y8))
    wq, _, _ = orc.hadamard_quant_act(x_bits)
    rng = np.random.default_rng(3)
    rows, cols = rng.integers(0, M, 2000), rng.integers(0, N, 2000)
    want = orc.int_gemm_sampled(wq, host(packed), K, rows, cols)
    np.testing.assert_array_equal(host(acc6)[rows, cols], want)
