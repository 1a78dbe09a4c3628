"""Seeded synthetic inputs for the weight-only quantized linear.

This module only draws random numbers and lays them out. It holds none of the
method's arithmetic (no quantisation, no dequantisation, no matmul), so both the
CPU oracle and the GPU path may take their inputs from it without sharing any
of the computation under test.

Workload recipe (the pages run real checkpoints; these stand in for them):

* W is fp32 [N, K] row-major (N = output channels, K = input features), every
  element N(0, 0.02^2).  The W4 group-128 workloads add outliers: each element
  independently, with probability 0.01, is multiplied by 8.
* x is bf16 [M, K]: fp32 N(0, 1) draws rounded to the nearest bf16 (ties to
  even), returned as raw uint16 bit patterns.

RNG: NumPy ``default_rng`` (PCG64).  W is drawn in row blocks of ``ROW_BLOCK``
rows; block b of a (cfg, K, N) weight uses the seed ``[cfg, K, N, b]`` so any
row range can be regenerated without drawing the rows before it.  Within a block
the normals are drawn first, then the outlier uniforms.  x uses the seed
``[cfg, K, M, 1]``.
"""
from __future__ import annotations

import numpy as np

ROW_BLOCK = 4096
W_STD = np.float32(0.02)
OUTLIER_P = np.float32(0.01)
OUTLIER_MUL = np.float32(8.0)


def _weight_block(cfg: int, K: int, N: int, b: int, outliers: bool) -> np.ndarray:
    r0 = b * ROW_BLOCK
    rows = min(ROW_BLOCK, N - r0)
    rng = np.random.default_rng([cfg, K, N, b])
    w = rng.standard_normal((rows, K), dtype=np.float32)
    w *= W_STD
    if outliers:
        mask = rng.random((rows, K), dtype=np.float32) < OUTLIER_P
        w[mask] *= OUTLIER_MUL
    return w


def weight_rows(cfg: int, K: int, N: int, r0: int, r1: int, outliers: bool = False) -> np.ndarray:
    """Rows [r0, r1) of the seeded fp32 weight W[N, K]."""
    if not (0 <= r0 <= r1 <= N):
        raise ValueError(f"row range [{r0},{r1}) outside [0,{N})")
    out = np.empty((r1 - r0, K), dtype=np.float32)
    b = r0 // ROW_BLOCK
    while b * ROW_BLOCK < r1:
        blk = _weight_block(cfg, K, N, b, outliers)
        s0 = max(r0, b * ROW_BLOCK)
        s1 = min(r1, b * ROW_BLOCK + blk.shape[0])
        out[s0 - r0:s1 - r0] = blk[s0 - b * ROW_BLOCK:s1 - b * ROW_BLOCK]
        b += 1
    return out


def weight(cfg: int, K: int, N: int, outliers: bool = False) -> np.ndarray:
    """The full seeded fp32 weight W[N, K] (row-major)."""
    return weight_rows(cfg, K, N, 0, N, outliers)


def _round_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern, nearest, ties to even (input preparation only)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    return (u >> np.uint64(16)).astype(np.uint16)


def activation(cfg: int, K: int, M: int) -> np.ndarray:
    """Seeded bf16 activations x[M, K] as uint16 bit patterns, x ~ N(0, 1)."""
    rng = np.random.default_rng([cfg, K, M, 1])
    return _round_to_bf16_bits(rng.standard_normal((M, K), dtype=np.float32))


def activation_f16(cfg: int, K: int, M: int) -> np.ndarray:
    """Seeded fp16 activations x[M, K] as uint16 bit patterns: the same N(0, 1) fp32
    draws as ``activation``, rounded to fp16 (nearest even) instead of bf16."""
    rng = np.random.default_rng([cfg, K, M, 1])
    return rng.standard_normal((M, K), dtype=np.float32).astype(np.float16).view(np.uint16)


def one_hot_activation(K: int, cols) -> np.ndarray:
    """bf16 bit patterns of x whose row m is the unit vector e_{cols[m]}."""
    cols = list(cols)
    x = np.zeros((len(cols), K), dtype=np.uint16)
    for m, k in enumerate(cols):
        x[m, k] = 0x3F80  # bf16 1.0
    return x


def identity_activation(K: int) -> np.ndarray:
    """bf16 bit patterns of the K x K identity."""
    x = np.zeros((K, K), dtype=np.uint16)
    x[np.arange(K), np.arange(K)] = 0x3F80
    return x


# The five workload families (K, N shapes and M values).
CONFIGS = {
    1: dict(name="w8pc_gemv_small", fmts=("w8pc",), shapes=[(1024, 1024)], Ms=[1]),
    2: dict(name="w8pc_gemv_decode", fmts=("w8pc",),
            shapes=[(5120, 27648), (13824, 5120), (5120, 7168), (6144, 5120)], Ms=[1, 2, 4, 7]),
    3: dict(name="w4g128_gemv_decode", fmts=("w4g128",),
            shapes=[(5120, 27648), (13824, 5120)], Ms=[1, 4]),
    4: dict(name="splitk_stress", fmts=("w8pc", "w8g128", "w4g128"),
            shapes=[(27648, 5120), (5120, 151936)], Ms=[1]),
    5: dict(name="prefill_gemm", fmts=("w8pc", "w4g128"),
            shapes=[(5120, 27648), (13824, 5120)], Ms=[8, 64, 512, 2048]),
}


def uses_outliers(fmt: str) -> bool:
    """W4 workloads carry the 1% x8 outliers; W8 workloads are plain Gaussian."""
    return fmt.startswith("w4")


def moe_offsets(seed: int, T: int, E: int, empty=()) -> np.ndarray:
    """Row offsets [E + 1] of T token rows grouped by E experts: a seeded random split
    (each row's expert drawn uniformly, counted per expert), the experts listed in
    `empty` left without rows.  Only the counts are drawn; the rows of x stay in the
    order the caller lays them out."""
    rng = np.random.default_rng([seed, T, E, 7])
    live = np.array([e for e in range(E) if e not in set(empty)], dtype=np.int64)
    pick = live[rng.integers(0, live.size, T)] if live.size else np.zeros(0, dtype=np.int64)
    counts = np.bincount(pick, minlength=E)
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
