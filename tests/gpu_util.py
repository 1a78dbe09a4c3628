"""Helpers shared by the GPU parity tests: seeded inputs on the device, packing
through the C ABI, and the oracle computed on the same host arrays."""
from __future__ import annotations

import functools

import numpy as np
import torch

import oracle.linear as OL
import oracle.quant as OQ
import synth

DEV = "cuda:0"


@functools.lru_cache(maxsize=4)
def host_weight(cfg: int, K: int, N: int, outliers: bool) -> np.ndarray:
    return synth.weight(cfg, K, N, outliers)


def to_dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def to_dev_bf16(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV)
    return t.view(torch.bfloat16)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def quantize_on_gpu(wq, W: np.ndarray, fmt: str):
    """wq_pack + wq_repack on the device; returns (gfx950 weight, canonical weight)."""
    Wt = to_dev_f32(W)
    g, can = wq.quantize(Wt, fmt, keep_canonical=True)
    del Wt
    return g, can


def canonical_to_host(can, fmt: str) -> dict:
    """Canonical device bytes -> the oracle's dict of arrays (for bit comparison)."""
    K, N = can.K, can.N
    q = can.qweight.cpu().numpy()
    s = can.scales.cpu().numpy()
    if fmt == "w8pc":
        return dict(fmt=fmt, K=K, N=N, qweight=q.view(np.int8).reshape(N, K), scales=s.view(np.uint16).reshape(N))
    if fmt.startswith("w8g"):
        G = K // int(fmt[3:])
        return dict(fmt=fmt, K=K, N=N, qweight=q.view(np.int8).reshape(N, K),
                    scales=s.view(np.uint16).reshape(N, G))
    z = can.zeros.cpu().numpy()
    if fmt == "w4pc":
        return dict(fmt=fmt, K=K, N=N, qweight=q.view(np.uint32).reshape(N, K // 8),
                    scales=s.view(np.float16).reshape(N), zeros=z.view(np.uint32).reshape(N // 8))
    G = K // int(fmt[3:])
    return dict(fmt=fmt, K=K, N=N, qweight=q.view(np.uint32).reshape(N, K // 8),
                scales=s.view(np.float16).reshape(N, G), zeros=z.view(np.uint32).reshape(G, N // 8))


def sample_rows(N: int, count: int = 64, seed: int = 0) -> np.ndarray:
    """8-aligned blocks of rows spread over [0, N) including both ends."""
    rng = np.random.default_rng(seed)
    blocks = N // 8
    pick = set([0, blocks - 1]) | set(rng.choice(blocks, size=min(blocks, max(2, count // 8)), replace=False).tolist())
    rows = np.concatenate([np.arange(8 * b, 8 * b + 8) for b in sorted(pick)])
    return rows[rows < N]


def oracle_pack_rows(fmt: str, W: np.ndarray, rows: np.ndarray) -> dict:
    """Oracle packing of the given rows only (rows come in whole 8-row blocks)."""
    return OQ.pack(fmt, W[rows])


def assert_parity(y_bits: np.ndarray, y_ref: np.ndarray, what: str) -> dict:
    st = OL.compare(y_bits, y_ref)
    assert st["fails"] == 0, f"{what}: {st}"
    # exact-code kernels show only the final bf16 rounding (about 0.39 of the bound)
    assert st["max_ratio"] < 0.6, f"{what}: error larger than bf16 output rounding: {st}"
    return st
