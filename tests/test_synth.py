"""The seeded input recipe (CPU only): the workload shapes, the seeds, the
bf16 rounding and the outlier channels are what the design notes state, and
every draw is reproducible."""
import numpy as np
import pytest

from bit_gemm_ternary_amd import synth


def test_workload_shapes():
    assert [(l.M, l.K, l.N) for l in synth.workload("tiny")] == [(4, 256, 512)]
    assert [(l.M, l.K, l.N) for l in synth.workload("decode")] == [(1, 4096, 4096), (1, 4096, 11008),
                                                                   (1, 11008, 4096)]
    assert [(l.M, l.K, l.N) for l in synth.workload("prefill")] == [(2048, 4096, 14336)]
    assert [(l.M, l.K, l.N) for l in synth.workload("hadamard")] == [(512, 4096, 4096), (512, 16384, 4096)]
    block = synth.workload("block", M=16)
    assert [(l.name, l.M, l.K, l.N) for l in block] == [
        ("q", 16, 4096, 4096), ("k", 16, 4096, 1024), ("v", 16, 4096, 1024), ("o", 16, 4096, 4096),
        ("gate", 16, 4096, 14336), ("up", 16, 4096, 14336), ("down", 16, 14336, 4096)]


def test_shard_is_the_block_cut_eight_ways():
    by = {l.name: l for l in synth.workload("block")}
    shard = {l.name: l for l in synth.workload("shard")}
    # split by output features: the rows of the grouped projections / 8, all of K
    assert shard["qkv/8"].N * 8 == by["q"].N + by["k"].N + by["v"].N and shard["qkv/8"].K == by["q"].K
    assert shard["gate_up/8"].N * 8 == by["gate"].N + by["up"].N and shard["gate_up/8"].K == by["gate"].K
    # split by input features: a K slice / 8, all rows; slices start at multiples of 64
    for name, full in (("o/8", "o"), ("down/8", "down")):
        assert shard[name].K * 8 == by[full].K and shard[name].N == by[full].N
        assert shard[name].K % 64 == 0
    assert all(l.M == 1 for l in shard.values())


def test_seeds_are_distinct_and_follow_the_rule():
    seeds = set()
    for name in ("tiny", "decode", "prefill", "hadamard", "block", "shard"):
        for l in synth.workload(name):
            s = [l.seed(r) for r in (0, 1, 2)]
            assert s == [1000 * synth.WORKLOAD_IDS[name] + 10 * l.layer_index + r for r in (0, 1, 2)]
            assert not seeds.intersection(s)
            seeds.update(s)


def test_draws_are_reproducible():
    l = synth.workload("decode")[1]
    np.testing.assert_array_equal(l.weights(), l.weights())
    np.testing.assert_array_equal(l.activations(), l.activations())
    assert l.weights().dtype == np.float32 and l.activations().dtype == np.uint16


@pytest.mark.parametrize("v,bits", [(1.0, 0x3F80), (-2.0, 0xC000), (0.0, 0x0000),
                                    (1.0 + 2.0 ** -8, 0x3F80),            # tie: to even (down)
                                    (1.0 + 3 * 2.0 ** -8, 0x3F82),        # tie: to even (up)
                                    (1.0 + 2.0 ** -8 + 2.0 ** -20, 0x3F81)])
def test_bf16_rounding_is_nearest_even(v, bits):
    assert int(synth.bf16_bits(np.array([v], np.float32))[0]) == bits


def test_outlier_channels():
    """round(frac * K) whole channels are scaled: with factor 1 the draw is the
    plain one, and the scaled channels are the ones that differ."""
    M, K = 3, 4096
    plain = synth.activations(M, K, 123, 124)
    scaled = synth.activations(M, K, 123, 124, outlier_frac=0.01, outlier_factor=20.0)
    differ = np.flatnonzero((plain != scaled).any(axis=0))
    assert len(differ) == round(0.01 * K)
    f = lambda b: (b.astype(np.uint32) << 16).view(np.float32)
    ratio = f(scaled[:, differ]) / f(plain[:, differ])
    assert np.allclose(ratio, 20.0, rtol=2 ** -7)
