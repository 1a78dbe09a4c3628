"""Top-k of LM-head logits and one token drawn from it (oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The tileInfer README's feature list names a fused LM head + top-k step (one kernel
for the logits and the sampling) and a top-k that only gathers the k best logits
across ranks ("Distributed Top-k Sampling").  The page states nothing more, so this
module fixes the plainest reading, which the library follows as well:

* the logits are the layer's own bf16 outputs, l[m, v] = bf16(x . dequant(W)^T)
  (``linear.ref_linear`` rounded to bf16, nearest even);
* top-k orders the vocabulary by logit value, larger first, and equal values by the
  smaller token index; -0 and +0 are equal values; a NaN logit ranks below every
  number; the first k entries are kept, in that order;
* sampling: with the kept logits v_1 >= ... >= v_k (tokens t_1 .. t_k), a
  temperature T > 0 and a uniform draw u in [0, 1) supplied by the caller, the
  weights are p_i = exp((v_i - v_1) / T) / sum_j exp((v_j - v_1) / T) and the token
  is t_j for the smallest j whose running sum p_1 + ... + p_j exceeds u (the last
  kept token if rounding leaves every sum at or below u); T = 0 takes t_1, and so
  does a best logit that is not finite (+inf dominates; -inf or NaN everywhere
  leaves nothing to weigh); a kept NaN logit behind a finite best one weighs 0.

Arithmetic here is fp64 on the bf16 values (exactly representable).
"""
from __future__ import annotations

import math

import numpy as np

from . import quant as _quant


def _values(bits) -> np.ndarray:
    """bf16 bit patterns -> fp64 values, with NaN kept as NaN."""
    with np.errstate(invalid="ignore"):
        return _quant.bf16_bits_to_f32(np.asarray(bits, dtype=np.uint16)).astype(np.float64)


def _rank_key(value: float, index: int):
    """Sort key of one vocabulary entry: numbers before NaN, the larger value first
    (-0 == +0), then the smaller index."""
    if math.isnan(value):
        return (1, 0.0, index)
    return (0, -value, index)


def _weight(v: float, v1: float, temperature: float) -> float:
    """Unnormalised probability of a kept logit v against the best one v1."""
    return math.exp((v - v1) / temperature)


def _reached(running: float, u: float) -> bool:
    """The draw stops at the first running sum that exceeds u."""
    return running > u


def topk_row(logit_bits, k: int):
    """Indices and bf16 bits of the k best logits of one row, best first (the order
    stated in the module docstring)."""
    b = np.asarray(logit_bits, dtype=np.uint16).ravel()
    V = b.size
    if not 1 <= k <= V:
        raise ValueError("need 1 <= k <= vocabulary size")
    val = _values(b)
    order = sorted(range(V), key=lambda i: _rank_key(float(val[i]), i))
    idx = np.array(order[:k], dtype=np.int64)
    return idx, b[idx]


def sample_row(kept_bits, kept_idx, temperature: float, u: float) -> int:
    """The token drawn from the kept logits (best first) with draw u in [0, 1)."""
    if temperature < 0 or not math.isfinite(temperature):
        raise ValueError("temperature must be finite and >= 0")
    if not 0.0 <= u < 1.0:
        raise ValueError("u must lie in [0, 1)")
    idx = [int(i) for i in kept_idx]
    v = _values(kept_bits)
    if temperature == 0 or not math.isfinite(float(v[0])):
        return idx[0]
    w = [0.0 if math.isnan(float(v[i])) else _weight(float(v[i]), float(v[0]), temperature)
         for i in range(len(idx))]
    total = math.fsum(w)
    run = 0.0
    for i, wi in enumerate(w):
        run += wi / total
        if _reached(run, u):
            return idx[i]
    return idx[-1]


def ref_topk_sample(logit_bits, k: int, temperature: float, u):
    """Every row of logit_bits [M][V] (bf16 bits): (indices [M][k], bf16 bits [M][k],
    tokens [M])."""
    L = np.asarray(logit_bits, dtype=np.uint16)
    M = L.shape[0]
    u = np.asarray(u, dtype=np.float64).ravel()
    idx = np.zeros((M, k), dtype=np.int64)
    bits = np.zeros((M, k), dtype=np.uint16)
    tok = np.zeros(M, dtype=np.int64)
    for m in range(M):
        idx[m], bits[m] = topk_row(L[m], k)
        tok[m] = sample_row(bits[m], idx[m], temperature, float(u[m]))
    return idx, bits, tok
