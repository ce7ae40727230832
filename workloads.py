"""Seeded synthetic inputs for the W4A16 workloads.

This module only draws random numbers and casts them to storage formats; it
holds none of the quantization or matmul arithmetic, and it is shared by the
tests, the benchmark and the smoke check on both sides of every comparison.

The pages quote their speed figures on 70B-parameter transformer layers; real
weights are not available here, so seeded normal weights with a few large input
channels stand in for them (large input channels are the outlier structure the
pages describe: a few channels set the range of a whole group).

Recipe (numpy PCG64, ``default_rng(seed)``):
  * weights: ``standard_normal(float32) * 0.02`` of shape [N][K]; a fraction of the
    input channels (columns k) chosen with ``rng.choice(K, n, replace=False)`` from
    a second seed is multiplied by 20 in every row; stored as bfloat16 (round to
    nearest even) or kept as float32;
  * activations: ``standard_normal(float32)`` of shape [M][K]; optionally 1% of the
    channels (the same ones in every row), chosen from a second seed, are
    multiplied by 10; stored as fp16 (round to nearest even);
  * seeds are ``1000 * c + t`` with c the workload number and t = 0 (weight
    values), 1 (weight outlier channels), 2 (activation values), 3 (activation
    outlier channels); for the sweep c = 50 + shape index and the activation seeds
    add 10 * log2(M).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Storage cast float32 -> bfloat16 bit patterns, round to nearest even
    (finite inputs only)."""
    u = np.ascontiguousarray(a, np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_f16_bits(a: np.ndarray) -> np.ndarray:
    """Storage cast float32 -> fp16 bit patterns, round to nearest even."""
    return np.asarray(a, np.float32).astype(np.float16).view(np.uint16)


def f16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return np.asarray(h, np.uint16).view(np.float16).astype(np.float32)


def gen_weights(seed: int, N: int, K: int, std: float = 0.02, outlier_frac: float = 0.0,
                outlier_mult: float = 20.0, dtype: str = "bf16") -> np.ndarray:
    """Weights [N][K]: float32 array (dtype "f32") or bfloat16 bit patterns ("bf16")."""
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((N, K), dtype=np.float32)
    w *= np.float32(std)
    n_out = int(round(outlier_frac * K))
    if n_out:
        cols = np.random.default_rng(seed + 1).choice(K, n_out, replace=False)
        w[:, cols] *= np.float32(outlier_mult)
    if dtype == "f32":
        return w
    if dtype == "bf16":
        return f32_to_bf16_bits(w)
    raise ValueError(dtype)


def gen_activations(seed: int, M: int, K: int, outlier_frac: float = 0.0,
                    outlier_mult: float = 10.0, channel_seed: int | None = None,
                    offset: float = 0.0) -> np.ndarray:
    """Activations [M][K] as fp16 bit patterns: N(offset, 1), then the outlier
    channels scaled by outlier_mult.  The outlier channels are drawn from
    channel_seed (default seed + 1), so draws with different values can share
    them (calibration rows and evaluation rows of one layer)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K), dtype=np.float32)
    if offset:
        x += np.float32(offset)
    n_out = int(round(outlier_frac * K))
    if n_out:
        cols = np.random.default_rng(seed + 1 if channel_seed is None else channel_seed).choice(K, n_out, replace=False)
        x[:, cols] *= np.float32(outlier_mult)
    return f32_to_f16_bits(x)


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    group: int
    w_seed: int
    x_seed: int
    w_dtype: str = "bf16"
    w_outlier_frac: float = 0.001
    x_outlier_frac: float = 0.01
    note: str = ""

    def weights(self) -> np.ndarray:
        return gen_weights(self.w_seed, self.N, self.K, outlier_frac=self.w_outlier_frac, dtype=self.w_dtype)

    def activations(self) -> np.ndarray:
        return gen_activations(self.x_seed, self.M, self.K, outlier_frac=self.x_outlier_frac)

    def algorithmic_bytes(self) -> int:
        """Bytes the product must move: 4-bit codes, fp16 scales, 4-bit zeros,
        fp16 activations and fp16 outputs."""
        nk = self.N * self.K
        return nk // 2 + 2 * nk // self.group + nk // (2 * self.group) + 2 * self.M * self.K + 2 * self.M * self.N

    def algorithmic_bytes_w8(self) -> int:
        """The same for int8 weights: 8-bit codes and fp16 scales, no zero-points."""
        nk = self.N * self.K
        return nk + 2 * nk // self.group + 2 * self.M * self.K + 2 * self.M * self.N

    def flops(self) -> int:
        return 2 * self.M * self.N * self.K


def _sweep():
    shapes = [(8192, 8192, "q/o proj"), (1024, 8192, "k/v proj"), (28672, 8192, "gate/up proj"),
              (8192, 28672, "down proj")]
    out = []
    for si, (N, K, what) in enumerate(shapes):
        c = 50 + si
        for M in (1, 8, 32, 128):
            t = 10 * int(math.log2(M))
            out.append(Workload(f"sweep_{what.split()[0].replace('/', '')}_M{M}", M, N, K, 32,
                                w_seed=1000 * c, x_seed=1000 * c + 2 + t,
                                note=f"70B-style {what}, group 32"))
    return out


WORKLOADS = {
    "tiny": Workload("tiny", 1, 256, 1024, 128, w_seed=1000, x_seed=1002, w_dtype="f32",
                     w_outlier_frac=0.0, x_outlier_frac=0.0, note="fp32 weights, no outliers"),
    "decode_gemv": Workload("decode_gemv", 1, 8192, 8192, 128, w_seed=2000, x_seed=2002,
                            note="M=1 decode GEMV"),
    "mlp_up_decode": Workload("mlp_up_decode", 16, 28672, 8192, 128, w_seed=3000, x_seed=3002,
                              note="M=16 MLP up-projection"),
    "batched_gemm": Workload("batched_gemm", 128, 28672, 8192, 128, w_seed=3000, x_seed=4002,
                             x_outlier_frac=0.0, note="M=128 GEMM, same weights as the M=16 up-projection"),
}
for _w in _sweep():
    WORKLOADS[_w.name] = _w


# The 8-weight example from the "Numerical example" section of the quantization
# post (input values only).
WORKED_EXAMPLE_W = [0.31, -0.12, 0.78, -0.05, 1.42, -0.91, 0.23, 0.66]
