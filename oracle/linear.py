"""Reference linear y = x . dequant(W)^T and the parity statistics (oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The layer is the weight-only quantised linear of the tileInfer README (feature
table, "INT8 Weight-Only Quantization"; "Key Optimizations"): bf16 activations
times int8 (or int4, Marlin benchmark page, "Validation and limits") weights
carrying scales; the same page's list also names FP16 activations, which carry
x and y in fp16 over the same weights.  Its plain definition, which every GPU kernel (GEMV, split-K,
GEMM) must reach up to fp32 summation order and the final bf16 rounding:

    y[m, n] = sum_k x[m, k] * Wd[n, k],   Wd = dequant(packed W)   (exact fp32)

evaluated here in fp64 with NumPy's matmul, chunked along N to bound memory.
"""
from __future__ import annotations

import numpy as np

from . import quant as _quant

TOL_REL = 1e-2          # |y - y_ref| <= TOL_REL * max(1, |y_ref|) per output element
GEMV_MAX_TOKENS = 7     # tokens < 8 -> GEMV, >= 8 -> GEMM


def token_count(x_shape) -> int:
    """numel(x) / x.shape[-1], the token count of the awq dispatch excerpt
    ("Heuristic: Mit han lab Llm awq Kernel Selection Thresholds", code from
    awq/quantize/qmodule.py)."""
    n = 1
    for d in x_shape:
        n *= int(d)
    return n // int(x_shape[-1])


def use_gemv(M: int) -> bool:
    """Same page, "The Insight (Rule of Thumb)", Linear Kernel: fewer than 8
    tokens take the GEMV kernel, 8 or more the GEMM kernel."""
    return M < GEMV_MAX_TOKENS + 1


ACTIVATIONS = ("bf16", "f16")


def f16_bits_to_f64(bits) -> np.ndarray:
    """fp16 bit patterns -> the values they denote (NumPy's IEEE binary16 decode, exact;
    subnormals, infinities and NaNs included)."""
    return np.ascontiguousarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def _x64(x_bits, act: str = "bf16") -> np.ndarray:
    """Activation bit patterns -> fp64 values: bf16 (the configs' activations) or fp16
    (the FP16 activations of the Marlin page's "Validation and limits" list)."""
    if act == "f16":
        return f16_bits_to_f64(x_bits)
    if act != "bf16":
        raise ValueError(f"unknown activation type {act!r}")
    return _quant.bf16_bits_to_f32(x_bits).astype(np.float64)


def ref_linear(x_bits: np.ndarray, P: dict, chunk: int = 4096, act: str = "bf16") -> np.ndarray:
    """fp64 y[M, N] for x[M, K] (uint16 bits of bf16, or of fp16 with act="f16") and a
    canonical packed weight.  The weight formats do not depend on the activation type:
    y is the same sum whichever 16-bit type carries x."""
    x = _x64(x_bits, act)
    N = P["N"]
    y = np.empty((x.shape[0], N), dtype=np.float64)
    for n0 in range(0, N, chunk):
        rows = np.arange(n0, min(N, n0 + chunk))
        Wd = _quant.dequant(P, rows).astype(np.float64)
        y[:, n0:n0 + len(rows)] = x @ Wd.T
    return y


def ref_linear_columns(x_bits: np.ndarray, P: dict, cols, act: str = "bf16") -> np.ndarray:
    """fp64 y[:, cols] only: the oracle one output channel at a time, for
    sampled checks at sizes where the full product is too slow on the host."""
    cols = np.asarray(cols)
    x = _x64(x_bits, act)
    Wd = _quant.dequant(P, cols).astype(np.float64)
    return x @ Wd.T


def ref_linear_residual(x_bits: np.ndarray, P: dict, r_bits: np.ndarray, act: str = "bf16") -> np.ndarray:
    """fp64 y = x . dequant(W)^T + r: the layer with the residual of its output added before
    the output is rounded (the fused residual of the tileInfer README's "Key
    Optimizations"; r in the activation type, [M, N])."""
    y = ref_linear(x_bits, P, act=act)
    r = _x64(np.asarray(r_bits, dtype=np.uint16).reshape(y.shape), act)
    return y + r


def gather_activations(x_bits: np.ndarray, perm) -> np.ndarray:
    """x'[m, j] = x[m, perm[j]] (bf16 bits), an index outside [0, K) giving +0: the
    full-K activation permutation that the Marlin register and launch scheduling
    benchmark page lists among its validated cases ("Validation and limits").  The
    stored weight then holds the columns in the same order, W'[n, j] = W[n, perm[j]],
    so that x' . W'^T = x . W^T when perm is a permutation."""
    x = np.asarray(x_bits, dtype=np.uint16)
    x = x.reshape(-1, x.shape[-1])
    K = x.shape[1]
    perm = np.asarray(perm, dtype=np.int64).ravel()
    if perm.size != K:
        raise ValueError("perm must hold K indices")
    out = np.zeros_like(x)
    for j, i in enumerate(perm):
        if 0 <= i < K:
            out[:, j] = x[:, i]
    return out


def ref_linear_perm(x_bits: np.ndarray, P: dict, perm) -> np.ndarray:
    """fp64 y = x' . dequant(W')^T with x' the activations gathered by perm."""
    return ref_linear(gather_activations(x_bits, perm), P)


def compare(y_bits: np.ndarray, y_ref: np.ndarray, act: str = "bf16") -> dict:
    """Per-element check of bf16 results (fp16 with act="f16") against the fp64
    reference.

    Returns max(err/tol), the number of failures and the relative RMS
    ||y - y_ref|| / ||y_ref|| (the statistic the Marlin benchmark page reports
    for its fixed-input projection check).  Over a zero reference that ratio is
    0 when y is zero as well and +inf otherwise.
    """
    y = _x64(y_bits, act)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    if y.shape != y_ref.shape:
        raise ValueError(f"shape mismatch {y.shape} vs {y_ref.shape}")
    err = np.abs(y - y_ref)
    tol = TOL_REL * np.maximum(1.0, np.abs(y_ref))
    ratio = err / tol
    num = float(np.sqrt(np.sum((y - y_ref) ** 2)))
    denom = float(np.sqrt(np.sum(y_ref * y_ref)))
    if denom > 0:
        rel_rms = num / denom
    else:
        rel_rms = 0.0 if num == 0 else float("inf")
    return dict(max_ratio=float(ratio.max()) if ratio.size else 0.0,
                fails=int(np.count_nonzero(ratio > 1.0)),
                rel_rms=rel_rms, n=int(ratio.size))
