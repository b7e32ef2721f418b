"""Seeded synthetic inputs for the BitLinear workloads.

This module only draws random numbers and converts float32 to bfloat16 bits; it
holds none of the method's arithmetic, so both the GPU path and the CPU oracle
can be fed from it.  numpy only (no torch, no GPU).

Workloads (shapes are M tokens, K in features, N out features; weights are
stored [N][K] as in a bias-free linear layer):

* ``tiny``     M=4, K=256, N=512; weights N(0, 0.02); activations N(0, 1)
               with 1% of channels scaled x20.
* ``decode``   M=1 and (K, N) in (4096, 4096), (4096, 11008), (11008, 4096);
               1% outlier channels x20.
* ``prefill``  M=2048, K=4096, N=14336; 0.5% outlier channels x50.
* ``hadamard`` M=512 and (K, N) in (4096, 4096), (16384, 4096); activations
               Student-t with 3 degrees of freedom.
* ``block``    the seven projections of a Llama-3-8B block (q 4096->4096,
               k/v 4096->1024, o 4096->4096, gate/up 4096->14336,
               down 14336->4096) at M in (1, 16, 256); activations N(0, 1).
* ``shard``    one device's share of that block split eight ways, M = 1:
               q|k|v and gate|up by output features (4096->768, 4096->3584),
               o and down by input features (512->4096, 1792->4096).

Seeds: ``seed = 1000 * workload_id + 10 * layer + role`` with role 0 for the
weights, 1 for the activations and 2 for the choice of outlier channels.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

WORKLOAD_IDS = {"tiny": 1, "decode": 2, "prefill": 3, "hadamard": 4, "block": 5, "shard": 6}

BLOCK_LAYERS = (  # name, K (in), N (out)
    ("q", 4096, 4096),
    ("k", 4096, 1024),
    ("v", 4096, 1024),
    ("o", 4096, 4096),
    ("gate", 4096, 14336),
    ("up", 4096, 14336),
    ("down", 14336, 4096),
)

SHARD_LAYERS = (  # name, K (in), N (out): the block cut eight ways
    ("qkv/8", 4096, 768),
    ("o/8", 512, 4096),
    ("gate_up/8", 4096, 3584),
    ("down/8", 1792, 4096),
)


@dataclass(frozen=True)
class Layer:
    """One BitLinear problem: shapes, activation recipe and seeds."""
    workload: str
    name: str
    M: int
    K: int
    N: int
    layer_index: int = 0
    act_dist: str = "normal"          # "normal" or "student_t"
    outlier_frac: float = 0.0
    outlier_factor: float = 1.0
    hadamard: bool = False

    def seed(self, role: int) -> int:
        return 1000 * WORKLOAD_IDS[self.workload] + 10 * self.layer_index + role

    def weights(self) -> np.ndarray:
        return weights(self.N, self.K, self.seed(0))

    def activations(self, M: int | None = None) -> np.ndarray:
        return activations(self.M if M is None else M, self.K, self.seed(1), self.seed(2),
                           dist=self.act_dist, outlier_frac=self.outlier_frac,
                           outlier_factor=self.outlier_factor)


def workload(name: str, M: int | None = None) -> list[Layer]:
    """The layers of one named workload (``M`` overrides the token count of ``block``)."""
    if name == "tiny":
        return [Layer("tiny", "tiny", 4, 256, 512, outlier_frac=0.01, outlier_factor=20.0)]
    if name == "decode":
        return [Layer("decode", f"{K}x{N}", 1, K, N, layer_index=i, outlier_frac=0.01,
                      outlier_factor=20.0)
                for i, (K, N) in enumerate(((4096, 4096), (4096, 11008), (11008, 4096)))]
    if name == "prefill":
        return [Layer("prefill", "ffn_up", 2048, 4096, 14336, outlier_frac=0.005,
                      outlier_factor=50.0)]
    if name == "hadamard":
        return [Layer("hadamard", f"{K}x{N}", 512, K, N, layer_index=i, act_dist="student_t",
                      hadamard=True)
                for i, (K, N) in enumerate(((4096, 4096), (16384, 4096)))]
    if name == "block":
        m = 1 if M is None else M
        return [Layer("block", lname, m, K, N, layer_index=i)
                for i, (lname, K, N) in enumerate(BLOCK_LAYERS)]
    if name == "shard":
        return [Layer("shard", lname, 1, K, N, layer_index=i)
                for i, (lname, K, N) in enumerate(SHARD_LAYERS)]
    raise KeyError(name)


def weights(N: int, K: int, seed: int, std: float = 0.02) -> np.ndarray:
    """float32 [N][K] weights drawn from N(0, std^2)."""
    rng = np.random.default_rng(seed)
    return rng.normal(0.0, std, (N, K)).astype(np.float32)


def activations(M: int, K: int, seed: int, outlier_seed: int | None = None, *,
                dist: str = "normal", outlier_frac: float = 0.0,
                outlier_factor: float = 1.0) -> np.ndarray:
    """bf16 activations [M][K] as uint16 bit patterns.

    Values are N(0, 1) (or Student-t with 3 degrees of freedom); then
    ``round(outlier_frac * K)`` channels, chosen without replacement, are
    multiplied by ``outlier_factor``; then each value is rounded to bf16.
    """
    rng = np.random.default_rng(seed)
    if dist == "normal":
        x = rng.standard_normal((M, K)).astype(np.float32)
    elif dist == "student_t":
        x = rng.standard_t(3, (M, K)).astype(np.float32)
    else:
        raise ValueError(dist)
    n_out = int(round(outlier_frac * K))
    if n_out:
        orng = np.random.default_rng(seed + 1 if outlier_seed is None else outlier_seed)
        idx = orng.choice(K, n_out, replace=False)
        x[:, idx] *= np.float32(outlier_factor)
    return bf16_bits(x)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_to_float(bits: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns -> float32 values (exact)."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
