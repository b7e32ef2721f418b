"""GPU checks of the row-parallel shard calls (Hugging Face 1.58-bit write-up,
"LLM을 1.58비트로 파인튜닝", section 양자화 메커니즘: the absmax and the RMS are
taken over the whole token; section 계산 패러다임: the contraction is integer
additions, so partial sums over K slices add up exactly).

One GPU stands in for G devices: the tokens, the gain and the packed weights
are cut into G K slices (contiguous copies, as each device would hold them);
the cross-device maximum and sum of the statistics and the sum of the int32
partials are done with torch here (they are the collective's job, not the
library's).  Every slice's codes must be the oracle's unsharded codes at those
positions and the summed partial accumulators the oracle's accumulators, bit
for bit; d_x and y within 1e-5 relative.
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


SHARD_CASES = [
    # (M, N, K, G, gain): the Llama-3-8B down and o projections cut eight ways
    # (K slices of 1792 and 512), the GEMV with several tokens, the skinny and
    # the tiled matrix-core paths, and two slices
    (1, 4096, 14336, 8, False),
    (1, 4096, 4096, 8, True),
    (4, 1001, 4096, 4, True),
    (16, 300, 8192, 8, False),
    (33, 700, 2048, 2, False),
]


@pytest.mark.parametrize("M,N,K,G,with_gain", SHARD_CASES)
def test_row_parallel_shards_reproduce_the_unsharded_layer(orc, dev, M, N, K, G, with_gain):
    print(f"case M={M} N={N} K={K} G={G} gain={with_gain}", flush=True)
    Ks = K // G
    x = synth.activations(M, K, 2800 + K % 97, 2801, outlier_frac=0.01, outlier_factor=20.0)
    if M > 2:
        x[1, :] = 0                                   # an all-zero token
    gain = np.random.default_rng(2802).uniform(0.5, 1.5, K).astype(np.float32) if with_gain else None
    packed, d_w, _, _ = orc.pack_weights(synth.weights(N, K, seed=2803))
    want_q, want_dx, _ = orc.quant_act(x, gain=gain)
    want_acc, want_y = orc.linear_forward(want_q, want_dx, packed, d_w, K)
    w_scale = to_dev(np.array([d_w, 0], np.float32), dev)

    xf = (x.astype(np.uint32) << 16).view(np.float32)
    u = xf * gain if gain is not None else xf
    xs = [bf16_to_dev(x[:, g * Ks:(g + 1) * Ks], dev) for g in range(G)]
    gs = [None if gain is None else to_dev(gain[g * Ks:(g + 1) * Ks], dev) for g in range(G)]
    stats = [bt.token_stats(xs[g], gs[g]) for g in range(G)]
    for g, (amax_g, ss_g) in enumerate(stats):
        sl = slice(g * Ks, (g + 1) * Ks)
        np.testing.assert_array_equal(host(amax_g), np.abs(u[:, sl]).max(axis=1))
        want_ss = (xf[:, sl].astype(np.float64) ** 2).sum(axis=1)
        np.testing.assert_allclose(host(ss_g), want_ss, rtol=1e-6, atol=0)

    # the collective's part: a maximum and a sum over the shards
    amax = torch.stack([a for a, _ in stats]).amax(dim=0)
    sumsq = torch.stack([s for _, s in stats]).sum(dim=0)

    acc = np.zeros((M, N), np.int64)
    scales = []
    for g in range(G):
        sl = slice(g * Ks, (g + 1) * Ks)
        xq_g, dx_g, qs_g = bt.quant_act_with_stats(xs[g], amax, sumsq, K, gain=gs[g])
        np.testing.assert_array_equal(host(xq_g), want_q[:, sl])
        np.testing.assert_array_equal(host(qs_g), want_q[:, sl].astype(np.int64).sum(axis=1))
        scales.append(host(dx_g))
        p_g = to_dev(packed[:, g * Ks // 4:(g + 1) * Ks // 4], dev)
        _, acc_g = bt.linear_forward(xq_g, dx_g, qs_g, p_g, w_scale, return_acc=True)
        acc += host(acc_g)
    for s in scales[1:]:
        np.testing.assert_array_equal(s, scales[0])       # one d_x on every shard
    assert_close_rel(scales[0], want_dx)
    if M > 2:
        assert scales[0][1] == 0
    np.testing.assert_array_equal(acc, want_acc)

    y = bt.dequant(to_dev(acc.astype(np.int32), dev), to_dev(scales[0], dev), w_scale)
    assert_close_rel(host(y), want_y)


@pytest.mark.parametrize("M,N,K", [(1, 4096, 4096), (3, 1001, 2048), (40, 512, 1024), (300, 1000, 512)])
def test_dequant_matches_the_contraction_epilogue(orc, dev, M, N, K):
    """bitnet_dequant of a contraction's own accumulators and d_x gives that
    contraction's y bit for bit (GEMV, skinny and tiled epilogues, N with and
    without 16-byte rows), and the oracle's y within 1e-5."""
    x = synth.activations(M, K, 2900 + M, 2901, outlier_frac=0.01, outlier_factor=20.0)
    packed, d_w, _, _ = orc.pack_weights(synth.weights(N, K, seed=2902))
    w_scale = to_dev(np.array([d_w, 0], np.float32), dev)
    xq, dx, qs = bt.quant_act(bf16_to_dev(x, dev))
    y, acc = bt.linear_forward(xq, dx, qs, to_dev(packed, dev), w_scale, return_acc=True)
    y2 = bt.dequant(acc, dx, w_scale)
    np.testing.assert_array_equal(host(y2), host(y))
    want_q, want_dx, _ = orc.quant_act(x)
    _, want_y = orc.linear_forward(want_q, want_dx, packed, d_w, K)
    assert_close_rel(host(y2), want_y)


def test_dequant_extreme_accumulators(dev):
    """Accumulators at the int32 extremes and zero: y = (float(acc) * d_x) * d_w
    in float32, zero for zero."""
    rng = np.random.default_rng(3000)
    M, N = 5, 4100
    acc = rng.integers(-2**31, 2**31, (M, N), dtype=np.int64).astype(np.int32)
    acc[0, :7] = [0, 1, -1, 2**31 - 1, -2**31, 2**24 + 1, -(2**24 + 3)]
    dx = rng.uniform(1e-4, 1e-2, M).astype(np.float32)
    dw = np.float32(0.0123)
    y = host(bt.dequant(to_dev(acc, dev), to_dev(dx, dev), to_dev(np.array([dw, 0], np.float32), dev)))
    want = (acc.astype(np.float32) * dx[:, None]) * dw    # float32 arithmetic, the same two roundings
    np.testing.assert_array_equal(y, want)
    assert y[0, 0] == 0


@pytest.mark.parametrize("M,K,with_gain", [(1, 4096, False), (5, 14336, True), (64, 512, False)])
def test_one_shard_is_the_unsharded_quantisation(dev, M, K, with_gain):
    """With a single shard the statistics pass and the quantisation from them
    reduce in the same order as bitnet_quant_act: codes, sums and d_x are
    bit-identical to it."""
    x = bf16_to_dev(synth.activations(M, K, 3100 + M, 3101, outlier_frac=0.01, outlier_factor=20.0), dev)
    gain = to_dev(np.random.default_rng(3102).uniform(0.5, 1.5, K).astype(np.float32), dev) if with_gain else None
    amax, sumsq = bt.token_stats(x, gain)
    q1, d1, s1 = bt.quant_act_with_stats(x, amax, sumsq, K, gain=gain)
    q0, d0, s0 = bt.quant_act(x, gain)
    np.testing.assert_array_equal(host(q1), host(q0))
    np.testing.assert_array_equal(host(s1), host(s0))
    np.testing.assert_array_equal(host(d1), host(d0))
