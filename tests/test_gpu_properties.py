"""GPU determinism, launch-configuration and property tests.

* Determinism: every entry point run ten times on the same inputs gives
  bit-identical outputs (a race in LDS or between waves would show up here).
* Launch configurations: the dispatcher picks kernels and launch shapes by
  M, N and K (GEMV with 256- or 512-thread groups and several batch sizes,
  skinny MFMA, three GEMM tilings, fused or not); the same rows computed under
  different choices must give identical int32 accumulators.
* Properties: power-of-two scaling of a token leaves its codes unchanged;
  permuting weight rows permutes the outputs; zero and single-spike tokens;
  random shapes (hypothesis) against the oracle, small ones through the fused
  path and larger ones through every tiling of the int8 and FP4 x FP6
  contractions; a rejected call leaves its outputs untouched.
"""
import ctypes

import numpy as np
import pytest
from hypothesis import HealthCheck, assume, given, settings, strategies as st

import bit_gemm_ternary_amd as bt
import f6_layout  # host encoder of the 6-bit activation layout
from bit_gemm_ternary_amd import synth

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


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


def weights_on(dev, N, K, seed, hadamard=False):
    return bt.pack_weights(to_dev(synth.weights(N, K, seed=seed), dev), hadamard=hadamard)


def tokens_on(dev, M, K, seed, dist="normal"):
    return bf16_to_dev(synth.activations(M, K, seed, seed + 1, dist=dist, outlier_frac=0.01,
                                         outlier_factor=20.0), dev)


# ---------------------------------------------------------------------------
# Determinism.
# ---------------------------------------------------------------------------

def _runs_identical(fn, n=20):
    first = [host(t) for t in fn()]
    for _ in range(n - 1):
        cur = [host(t) for t in fn()]
        for a, b in zip(first, cur):
            np.testing.assert_array_equal(a, b)


def test_every_entry_point_is_deterministic(dev):
    K, N = 4096, 1024
    W = to_dev(synth.weights(N, K, seed=800), dev)
    packed, ws = bt.pack_weights(W)
    x1 = tokens_on(dev, 1, K, 801)
    x16 = tokens_on(dev, 16, K, 803)
    x512 = tokens_on(dev, 512, K, 805)
    _runs_identical(lambda: bt.pack_weights(W))
    _runs_identical(lambda: bt.pack_weights(W, hadamard=True))
    _runs_identical(lambda: bt.quant_act(x512))
    _runs_identical(lambda: bt.hadamard_quant_act(x512))
    _runs_identical(lambda: bt.hadamard_quant_act_f6(x512))
    for x in (x1, x16, x512):  # GEMV, skinny MFMA, GEMM
        q, dx, qs = bt.quant_act(x)
        _runs_identical(lambda: bt.linear_forward(q, dx, qs, packed, ws, return_acc=True))
    _runs_identical(lambda: (bt.bitlinear_forward(x1, packed, ws),))
    ph, wh = bt.pack_weights(W, hadamard=True)
    q6, dx6, qs6 = bt.hadamard_quant_act_f6(x512)
    _runs_identical(lambda: bt.linear_forward_f6(q6, dx6, qs6, ph, wh, return_acc=True))
    _runs_identical(lambda: bt.hadamard_quant_act_i4(x512))
    q4, dx4, qs4 = bt.hadamard_quant_act_i4(x512)
    for m in (1, 4, 16, 512):  # nibble GEMV, nibble tiles
        _runs_identical(lambda: bt.linear_forward_i4(q4[:m], dx4[:m], qs4[:m], ph, wh, return_acc=True))
    _runs_identical(lambda: (bt.linear_forward_blend(x16, W, packed, ws, 0.5),))
    gy = bf16_to_dev(synth.bf16_bits(np.random.default_rng(807).standard_normal((512, N)).astype(np.float32)), dev)
    pt = bt.transpose_packed(packed, K)
    q, dx, _ = bt.quant_act(x512)
    _runs_identical(lambda: (bt.transpose_packed(packed, K),))
    _runs_identical(lambda: (bt.linear_backward_input(gy, pt, ws),))
    _runs_identical(lambda: (bt.linear_backward_weight(gy, q, dx),))
    gn = bt.linear_backward_input(gy, pt, ws)
    _runs_identical(lambda: bt.rmsnorm_backward(x512, gn, with_gain_grad=True))


# ---------------------------------------------------------------------------
# Launch configurations agree.
# ---------------------------------------------------------------------------

def test_token_counts_across_kernels_agree(dev):
    # the first rows through the GEMV (M <= 4), the skinny kernel (M <= 16) and
    # the GEMM tilings (64x64 at small M; 128x128 at N = 4096 and 448x128 at
    # N = 14336 for M = 2048) must equal the M = 2048 result row for row
    K = 4096
    for N in (4096, 14336):
        packed, ws = weights_on(dev, N, K, 810 + N % 7)
        q, dx, qs = bt.quant_act(tokens_on(dev, 2048, K, 812))
        _, ref = bt.linear_forward(q, dx, qs, packed, ws, return_acc=True)
        ref = host(ref)
        for M in (1, 2, 3, 4, 5, 16, 17, 64, 300):
            _, acc = bt.linear_forward(q[:M].contiguous(), dx[:M].contiguous(), qs[:M].contiguous(),
                                       packed, ws, return_acc=True)
            np.testing.assert_array_equal(host(acc), ref[:M])


def test_nibble_token_counts_across_kernels_agree(dev):
    # packed 4-bit codes: the first rows through the dot8 GEMV (M <= 4) and the
    # tile configurations equal the M = 512 result row for row, and all equal
    # the int8-container path on the same codes
    K, N = 4096, 4096
    W = to_dev(synth.weights(N, K, seed=815), dev)
    ph, wh = bt.pack_weights(W, hadamard=True)
    x = tokens_on(dev, 512, K, 816)
    q4, dx, qs = bt.hadamard_quant_act_i4(x)
    q8, _, _ = bt.hadamard_quant_act(x)
    _, ref = bt.linear_forward_i4(q4, dx, qs, ph, wh, return_acc=True)
    ref = host(ref)
    _, ref8 = bt.linear_forward(q8, dx, qs, ph, wh, return_acc=True)
    np.testing.assert_array_equal(ref, host(ref8))
    for M in (1, 2, 3, 4, 5, 16, 17, 64, 300):
        _, acc = bt.linear_forward_i4(q4[:M].contiguous(), dx[:M].contiguous(), qs[:M].contiguous(),
                                      ph, wh, return_acc=True)
        np.testing.assert_array_equal(host(acc), ref[:M])


def test_fused_and_standalone_decode_agree(dev):
    K = 11008
    packed, ws = weights_on(dev, 4096, K, 820)
    for M in (1, 2, 4):
        x = tokens_on(dev, M, K, 821 + M)
        y_f, codes, acc_f = _fused(dev, x, packed, ws)
        q, dx, qs = codes
        y_s, acc_s = bt.linear_forward(q, dx, qs, packed, ws, return_acc=True)
        np.testing.assert_array_equal(host(acc_f), host(acc_s))
        np.testing.assert_array_equal(host(y_f), host(y_s))


def _fused(dev, x, packed, ws):
    M, K = x.shape
    N = packed.shape[0]
    q = torch.empty((M, K), dtype=torch.int8, device=dev)
    dx = torch.empty(M, dtype=torch.float32, device=dev)
    qs = torch.empty(M, dtype=torch.int32, device=dev)
    acc = torch.empty((M, N), dtype=torch.int32, device=dev)
    y, _ = bt.bitlinear_forward(x, packed, ws, codes=(q, dx, qs), acc_out=acc)
    return y, (q, dx, qs), acc


@pytest.mark.parametrize("K,Ns", [(4096, (4096, 8192, 28672)), (11008, (1024, 4096, 8192, 10240))])
def test_decode_launch_shapes_agree(dev, K, Ns):
    # Rows of one packed matrix under different launch shapes: for K = 4096,
    # 256-thread groups with 4 rows per wave (N 4096), 512-thread groups with 4
    # rows per wave (N 8192) and, two per CU, 7 rows per wave (N 28672); for
    # K = 11008 (3 chunks per lane)
    # 256-thread groups (N 1024), 512-thread groups with 2 and 4 rows per wave,
    # and 5 rows per wave in two alternating register sets (N 10240).  The
    # first 1024 rows must come out the same every time.
    packed, ws = weights_on(dev, Ns[-1], K, 830 + K % 11)
    x = tokens_on(dev, 1, K, 831)
    ref = None
    for N in Ns:
        _, _, acc = _fused(dev, x, packed[:N].contiguous(), ws)
        a = host(acc)[:, :1024]
        if ref is None:
            ref = a
        else:
            np.testing.assert_array_equal(a, ref)


# ---------------------------------------------------------------------------
# Properties.
# ---------------------------------------------------------------------------

def test_power_of_two_scaling_keeps_codes(dev):
    K = 4096
    bits = synth.activations(4, K, 840, 841, outlier_frac=0.01, outlier_factor=20.0)
    x = synth.bf16_to_float(bits)
    # eps = 0: then d_x = amax / rms is scale free too, and float64 scales exactly
    q0, d0, s0 = (host(t) for t in bt.quant_act(bf16_to_dev(bits, dev), None, 0.0))
    for j in (-8, -1, 3, 20):
        scaled = synth.bf16_bits(x * np.float32(2.0 ** j))  # exact: bf16 keeps its mantissa
        q, d, s = (host(t) for t in bt.quant_act(bf16_to_dev(scaled, dev), None, 0.0))
        np.testing.assert_array_equal(q, q0)
        np.testing.assert_array_equal(s, s0)
        np.testing.assert_array_equal(d, d0)


def test_permuting_weight_rows_permutes_outputs(dev):
    K, N, M = 4096, 512, 33
    W = synth.weights(N, K, seed=842)
    perm = np.random.default_rng(843).permutation(N)
    packed, ws = bt.pack_weights(to_dev(W, dev))
    packed_p = packed[torch.from_numpy(perm).to(dev)].contiguous()
    q, dx, qs = bt.quant_act(tokens_on(dev, M, K, 844))
    y = host(bt.linear_forward(q, dx, qs, packed, ws))
    y_p = host(bt.linear_forward(q, dx, qs, packed_p, ws))
    np.testing.assert_array_equal(y_p, y[:, perm])


def test_zero_and_spike_tokens(orc, dev):
    K, N = 4096, 1024
    bits = np.zeros((3, K), np.uint16)
    bits[1, 1234] = synth.bf16_bits(np.array([-3.5], np.float32))[0]   # one spike
    bits[2] = synth.bf16_bits(np.full(K, 0.25, np.float32))            # constant token
    packed, ws = weights_on(dev, N, K, 845)
    y, (q, dx, qs), acc = _fused(dev, bf16_to_dev(bits, dev), packed, ws)
    q, dx, y = host(q), host(dx), host(y)
    assert (q[0] == 0).all() and dx[0] == 0 and (y[0] == 0).all()
    assert q[1, 1234] == -127 and np.count_nonzero(q[1]) == 1
    assert (q[2] == 127).all()
    wq, wdx, _ = orc.quant_act(bits)
    np.testing.assert_array_equal(q, wq)


def test_rejected_call_leaves_outputs_untouched(dev):
    K, N, M = 256, 64, 4
    q = torch.zeros((M, K), dtype=torch.int8, device=dev)
    dx = torch.ones(M, dtype=torch.float32, device=dev)
    qs = torch.zeros(M, dtype=torch.int32, device=dev)
    packed = torch.full((N, K // 4), 0x55, dtype=torch.uint8, device=dev)
    ws = torch.ones(2, dtype=torch.float32, device=dev)
    y = torch.full((M, N), 7.5, dtype=torch.float32, device=dev)
    L = bt.lib()
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    # K = 100 is not a multiple of 64: rejected before anything is enqueued
    assert L.bitnet_linear_forward(p(q), p(dx), p(qs), p(packed), p(ws), M, N, 100, p(y), None, stream) == 2
    # misaligned codes pointer
    assert L.bitnet_linear_forward(ctypes.c_void_p(q.data_ptr() + 1), p(dx), p(qs), p(packed), p(ws), M, N, K,
                                   p(y), None, stream) == 4
    assert (host(y) == 7.5).all()


@settings(max_examples=30, deadline=None, suppress_health_check=[HealthCheck.function_scoped_fixture])
@given(M=st.integers(1, 70), N=st.integers(1, 300), k64=st.integers(1, 20), seed=st.integers(0, 10 ** 6))
def test_random_small_shapes_match_the_oracle(orc, dev, M, N, k64, seed):
    K = 64 * k64
    W = synth.weights(N, K, seed=seed)
    bits = synth.activations(M, K, seed + 1, seed + 2, outlier_frac=0.02, outlier_factor=10.0)
    want_packed, d_w, _, _ = orc.pack_weights(W)
    wq, wdx, wqs = orc.quant_act(bits)
    want_acc, want_y = orc.linear_forward(wq, wdx, want_packed, d_w, K)
    packed, ws = bt.pack_weights(to_dev(W, dev))
    y, (q, dx, qs), acc = _fused(dev, bf16_to_dev(bits, dev), packed, ws) if M <= 4 else \
        (None, bt.quant_act(bf16_to_dev(bits, dev)), None)
    if acc is None:
        y, acc = bt.linear_forward(q, dx, qs, packed, ws, return_acc=True)
    np.testing.assert_array_equal(host(packed), want_packed)
    np.testing.assert_array_equal(host(q), wq)
    np.testing.assert_array_equal(host(acc), want_acc)
    got = host(y).astype(np.float64)
    assert np.all(np.abs(got - want_y) <= 1e-5 * np.abs(want_y))


@settings(max_examples=25, deadline=None, suppress_health_check=[HealthCheck.function_scoped_fixture])
@given(M=st.integers(1, 4), N=st.integers(1, 12000), k64=st.integers(1, 200), seed=st.integers(0, 10 ** 6))
def test_random_nibble_gemv_shapes_match_the_oracle(orc, dev, M, N, k64, seed):
    K = 64 * k64
    rng = np.random.default_rng(seed)
    W = synth.weights(N, K, seed=seed)
    packed, d_w, _, _ = orc.pack_weights(W)
    codes = rng.integers(-8, 8, (M, K)).astype(np.int8)
    d_x = rng.uniform(1e-3, 1e-2, M).astype(np.float32)
    qsum = codes.astype(np.int64).sum(axis=1).astype(np.int32)
    want_acc, want_y = orc.linear_forward(codes, d_x, packed, d_w, K)
    y, acc = bt.linear_forward_i4(to_dev(orc.pack_nibbles(codes), dev), to_dev(d_x, dev), to_dev(qsum, dev),
                                  to_dev(packed, dev), to_dev(np.array([d_w, 0], np.float32), dev),
                                  return_acc=True)
    np.testing.assert_array_equal(host(acc), want_acc)
    got = host(y).astype(np.float64)
    assert np.all(np.abs(got - want_y) <= 1e-5 * np.abs(want_y))


@settings(max_examples=25, deadline=None, suppress_health_check=[HealthCheck.function_scoped_fixture])
@given(M=st.integers(5, 700), N=st.integers(1, 4000), k64=st.integers(1, 260), fmt=st.sampled_from(["i8", "f6", "i4"]),
       seed=st.integers(0, 10 ** 6))
def test_random_tiled_shapes_match_the_oracle(orc, dev, M, N, k64, fmt, seed):
    # The tiled paths at random shapes: skinny (M <= 16), the 64 x 64 tiles in
    # one, two or four K groups, 128 x 64 tiles in three, the 256-row tiles;
    # ragged M, N and K (K need not fill the last 256-deep stage); int8, E3M2
    # and packed 4-bit codes.
    K = 64 * k64
    f6 = fmt != "i8"
    assume(M * N * K <= 2_500_000_000)
    rng = np.random.default_rng(seed)
    W = synth.weights(N, K, seed=seed)
    packed, d_w, _, _ = orc.pack_weights(W)
    lo, hi = (-8, 8) if f6 else (-127, 128)
    codes = rng.integers(lo, hi, (M, K)).astype(np.int8)
    d_x = rng.uniform(1e-3, 1e-2, M).astype(np.float32)
    qsum = codes.astype(np.int64).sum(axis=1).astype(np.int32)
    want_acc, want_y = orc.linear_forward(codes, d_x, packed, d_w, K)
    args = (to_dev(d_x, dev), to_dev(qsum, dev), to_dev(packed, dev),
            to_dev(np.array([d_w, 0], np.float32), dev))
    if fmt == "f6":
        y, acc = bt.linear_forward_f6(to_dev(f6_layout.encode(codes), dev), *args, return_acc=True)
    elif fmt == "i4":
        y, acc = bt.linear_forward_i4(to_dev(orc.pack_nibbles(codes), dev), *args, return_acc=True)
    else:
        y, acc = bt.linear_forward(to_dev(codes, dev), *args, return_acc=True)
    np.testing.assert_array_equal(host(acc), want_acc)
    got = host(y).astype(np.float64)
    assert np.all(np.abs(got - want_y) <= 1e-5 * np.abs(want_y))


# ---------------------------------------------------------------------------
# The layer against the dense computation it replaces (smoke checks of the
# method, not parity: ternary weights cost ~0.5 relative error by themselves).
# ---------------------------------------------------------------------------

def _dense(W, bits, eps=1e-5):
    """RMSNorm(x) @ W^T in float64."""
    x = synth.bf16_to_float(bits).astype(np.float64)
    n = x / np.sqrt((x * x).mean(axis=1, keepdims=True) + eps)
    return n @ W.astype(np.float64).T


def _rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def test_bitlinear_tracks_the_dense_layer(dev):
    M, K, N = 64, 4096, 1024
    W = synth.weights(N, K, seed=870)
    bits = synth.activations(M, K, 871, 872)
    packed, ws = bt.pack_weights(to_dev(W, dev))
    y = host(bt.bitlinear_forward(bf16_to_dev(bits, dev), packed, ws)).astype(np.float64)
    ref = _dense(W, bits)
    cos = float((y * ref).sum() / np.linalg.norm(y) / np.linalg.norm(ref))
    assert 0.85 <= cos <= 0.92, cos
    assert 0.45 <= _rel(y, ref) <= 0.56


def test_hadamard_lowers_the_int4_error_on_heavy_tails(orc, dev):
    # Student-t (3 degrees of freedom) tokens: int4 codes of the raw token lose
    # more than int4 codes of its Hadamard transform (the H-BitLinear premise).
    M, K, N = 64, 4096, 1024
    W = synth.weights(N, K, seed=873)
    bits = synth.activations(M, K, 874, 875, dist="student_t")
    ref = _dense(W, bits)
    # H path on the GPU
    packed, ws = bt.pack_weights(to_dev(W, dev), hadamard=True)
    q, dx, qs = bt.hadamard_quant_act(bf16_to_dev(bits, dev))
    y_h = host(bt.linear_forward(q, dx, qs, packed, ws)).astype(np.float64)
    # int4 codes without the transform, on the CPU, from the oracle's ternary weights
    _, d_w, _, qw = orc.pack_weights(W)
    x = synth.bf16_to_float(bits).astype(np.float64)
    a = np.abs(x).max(axis=1, keepdims=True)
    codes = np.clip(np.rint(x * (7.0 / a)), -8, 7)
    rstd = 1.0 / np.sqrt((x * x).mean(axis=1, keepdims=True) + 1e-5)
    y_plain = (codes @ qw.astype(np.float64).T) * (a * rstd / 7.0) * float(d_w)
    e_h, e_plain = _rel(y_h, ref), _rel(y_plain, ref)
    assert e_h < e_plain - 0.05, (e_h, e_plain)
    assert 0.45 <= e_h <= 0.60, e_h
