"""Grouped (mixture-of-experts) weight-only linear and the SiLU-gated product (oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The Marlin register and launch scheduling benchmark page ("Validation and limits")
validates a shared MoE kernel beside its dense one, and the SGLang quantization-stack
review (Figure 4 comments) argues for one shared WnA16 kernel across formats; the
tileInfer README's "Key Optimizations" list fuses the SiLU gate into the projection
that produces it.  None of them spells the arithmetic out, so the plain reading is
fixed here:

* E experts share one format and shape (K, N); the token rows of x are grouped by
  expert, expert e owning rows offsets[e] .. offsets[e + 1] - 1, and
      y[t, :] = x[t, :] . dequant(W_e)^T      for every row t of expert e
  -- the dense layer (``linear.ref_linear``) applied per expert to its own rows;
* the gated product of a fused gate/up projection (N = 2 I: gate rows first, then up
  rows) is  h[t, j] = silu(g[t, j]) * u[t, j]  with g = y[:, :I], u = y[:, I:] and
  silu(v) = v / (1 + exp(-v)) (v times the logistic sigmoid of v).

Arithmetic is fp64, as in the dense oracle.
"""
from __future__ import annotations

import numpy as np

from . import linear as _linear


def silu(v):
    """v / (1 + exp(-v)) elementwise, in fp64 (exp(-v) overflowing to inf gives -0.0 / 0.0)."""
    v = np.asarray(v, dtype=np.float64)
    with np.errstate(over="ignore"):
        return v / (1.0 + np.exp(-v))


def check_offsets(offsets, T: int) -> np.ndarray:
    """offsets[E + 1]: nondecreasing, starting at 0 and ending at T."""
    off = np.asarray(offsets, dtype=np.int64).ravel()
    if off.size < 2 or off[0] != 0 or off[-1] != T or np.any(np.diff(off) < 0):
        raise ValueError("offsets must rise from 0 to the row count")
    return off


def ref_moe_linear(x_bits, offsets, packed) -> np.ndarray:
    """fp64 y [T, N]: expert e's packed weight applied to its rows of x (bf16 bits [T, K])."""
    x = np.asarray(x_bits, dtype=np.uint16)
    T = x.shape[0]
    off = check_offsets(offsets, T)
    if len(packed) != off.size - 1:
        raise ValueError("one packed weight per expert")
    N = packed[0]["N"]
    y = np.zeros((T, N), dtype=np.float64)
    for e, P in enumerate(packed):
        r0, r1 = int(off[e]), int(off[e + 1])
        if r1 > r0:
            y[r0:r1] = _linear.ref_linear(x[r0:r1], P)
    return y


def silu_mul(y) -> np.ndarray:
    """h = silu(gate) * up for y = [gate | up] along the last axis (fp64)."""
    y = np.asarray(y, dtype=np.float64)
    n = y.shape[-1]
    if n % 2:
        raise ValueError("a fused gate/up output has an even width")
    i = n // 2
    return silu(y[..., :i]) * y[..., i:]


def ref_moe_silu_mul(x_bits, offsets, packed) -> np.ndarray:
    """fp64 h [T, N / 2] = silu_mul of the grouped gate/up projection."""
    return silu_mul(ref_moe_linear(x_bits, offsets, packed))


def ref_linear_silu_mul(x_bits, P) -> np.ndarray:
    """The dense layer's gated product: silu_mul(x . dequant(W)^T)."""
    return silu_mul(_linear.ref_linear(x_bits, P))


__all__ = ["silu", "check_offsets", "ref_moe_linear", "silu_mul", "ref_moe_silu_mul", "ref_linear_silu_mul"]
