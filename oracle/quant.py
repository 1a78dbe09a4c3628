"""Quantisers, canonical packed layouts and dequantisation (oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages name the formats but print no quantisation recipe, so this module
spells out the plain reading used throughout (each step below is one line of
NumPy, in the order the recipe states it):

Shared rules: all arithmetic is IEEE fp32, round to nearest with ties to even
(``np.rint``); bf16 and fp16 conversions round to nearest even.

W8, one scale per group of G consecutive k (G = K: per output channel, the
tileInfer README's "INT8 Weight-Only Quantization" feature; G = 128: the
group-128 INT8 head of the Marlin benchmark page, "Full inference"):
  1. a = max |w| over the group
  2. s = bf16(a / 127)                              -- the stored scale
  3. q = 0 if s == 0 else clamp(rint(w / s), -127, 127), dividing by the
     stored (rounded) scale
  layout: q int8 [N, K] row-major; s bf16 [N, K/G].

W8 also takes groups of 32 and 64 (the same three steps with G = 32 or 64: the
Marlin page's "Validation and limits" lists per-channel scales and groups of 32, 64
and 128): layout q int8 [N, K] row-major; s bf16 [N, K/G].

W4 asymmetric, one scale and zero-point per group of G consecutive k (G = 128:
INT4 + group 128; G = 32 or 64: the smaller groups of the same list; G = K: INT4
per output channel -- all in the Marlin page's "Validation and limits", which lists
INT4 with per-channel and group scales):
  1. hi = max w, lo = min w over the group
  2. s = fp16((hi - lo) / 15)                       -- the stored scale
  3. if s == 0: z = 0, q = 0
     else z = clamp(rint(-lo / s), 0, 15); q = clamp(rint(w / s) + z, 0, 15)
  layout: qweight uint32 [N, K/8], bits 4j..4j+3 of word (n, c) hold q[n, 8c+j];
          group G (32, 64, 128): scales fp16 [N, K/G];
                       zeros uint32 [K/G, N/8], bits 4j..4j+3 of word (g, c) hold z[8c+j, g];
          per channel: scales fp16 [N]; zeros uint32 [N/8], bits 4j..4j+3 of word c
                       hold z[8c+j] (the group-128 layout with one group).

Dequantisation is exact in fp32: W8 q*s, W4 (q - z)*s.
"""
from __future__ import annotations

import numpy as np

GROUP = 128
FORMATS = ("w8pc", "w8g128", "w4g128")
W4PC = "w4pc"  # INT4 per output channel (tested on its own; FORMATS are the configs' formats)
# every grouped format and its group size along K (the g32 / g64 variants are tested on
# their own, like W4PC)
GROUPED = {"w8g32": 32, "w8g64": 64, "w8g128": 128, "w4g32": 32, "w4g64": 64, "w4g128": 128}
SMALL_GROUPS = ("w8g32", "w8g64", "w4g32", "w4g64")


# ---------------------------------------------------------------- conversions
def bf16_rne_bits(a) -> np.ndarray:
    """fp32 -> bf16 bit pattern: add 0x7FFF plus bit 16, keep the top 16 bits.

    Nearest, ties to even, for every finite input (no NaNs occur here).
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    return ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    """bf16 bit pattern -> the fp32 value it denotes (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ----------------------------------------------------------------- quantisers
def _groups(W: np.ndarray, G: int) -> np.ndarray:
    W = np.ascontiguousarray(W, dtype=np.float32)
    N, K = W.shape
    if K % G:
        raise ValueError(f"K={K} is not a multiple of the group size {G}")
    return W.reshape(N, K // G, G)


def quantize_w8(W: np.ndarray, G: int | None = None):
    """Symmetric int8 quantisation with one bf16 scale per group of G along K.

    G=None means one group per output channel (G = K).
    Returns (q int8 [N, K], s_bits uint16 [N, K/G]).
    """
    W = np.ascontiguousarray(W, dtype=np.float32)
    N, K = W.shape
    G = K if G is None else G
    Wg = _groups(W, G)
    a = np.max(np.abs(Wg), axis=2)                        # step 1
    s_bits = bf16_rne_bits(a / np.float32(127.0))         # step 2
    s = bf16_bits_to_f32(s_bits)
    q = np.zeros(Wg.shape, dtype=np.float32)              # step 3
    nz = s != 0
    q[nz] = np.clip(np.rint(Wg[nz] / s[nz][:, None]), -127, 127)
    return q.astype(np.int8).reshape(N, K), s_bits


def quantize_w4(W: np.ndarray, G: int | None = GROUP):
    """Asymmetric uint4 quantisation, one fp16 scale and uint4 zero per group of G
    along K (G=None: one group per output channel, G = K).

    Returns unpacked (q uint8 [N, K] in 0..15, s fp16 [N, K/G], z uint8 [N, K/G]).
    """
    W = np.ascontiguousarray(W, dtype=np.float32)
    N, K = W.shape
    Wg = _groups(W, K if G is None else G)
    hi = np.max(Wg, axis=2)                                # step 1
    lo = np.min(Wg, axis=2)
    s16 = ((hi - lo) / np.float32(15.0)).astype(np.float16)  # step 2
    s = s16.astype(np.float32)
    z = np.zeros(s.shape, dtype=np.float32)                # step 3
    q = np.zeros(Wg.shape, dtype=np.float32)
    nz = s != 0
    z[nz] = np.clip(np.rint(-lo[nz] / s[nz]), 0, 15)
    q[nz] = np.clip(np.rint(Wg[nz] / s[nz][:, None]) + z[nz][:, None], 0, 15)
    return q.astype(np.uint8).reshape(N, K), s16, z.astype(np.uint8)


def quantize_w4g128(W: np.ndarray):
    """quantize_w4 with groups of 128 along K."""
    return quantize_w4(W, GROUP)


# -------------------------------------------------------------------- packing
def _pack_nibbles_rows(v: np.ndarray) -> np.ndarray:
    """[R, 8C] codes 0..15 -> [R, C] uint32; code 8c+j goes to bits 4j..4j+3 of word c."""
    R, L = v.shape
    v = v.astype(np.uint32).reshape(R, L // 8, 8)
    out = np.zeros((R, L // 8), dtype=np.uint32)
    for j in range(8):
        out |= v[:, :, j] << np.uint32(4 * j)
    return out


def _unpack_nibbles_rows(words: np.ndarray) -> np.ndarray:
    R, C = words.shape
    out = np.empty((R, C, 8), dtype=np.uint8)
    for j in range(8):
        out[:, :, j] = (words >> np.uint32(4 * j)) & np.uint32(0xF)
    return out.reshape(R, C * 8)


def pack(fmt: str, W: np.ndarray) -> dict:
    """Quantise W[N, K] (fp32) and lay the result out in the canonical packed form.

    Returns a dict of NumPy arrays holding exactly the bytes the canonical layout
    defines: ``qweight`` and ``scales`` (and ``zeros`` for W4).
    """
    W = np.ascontiguousarray(W, dtype=np.float32)
    N, K = W.shape
    if fmt == "w8pc":
        q, s = quantize_w8(W, None)
        return dict(fmt=fmt, K=K, N=N, qweight=q, scales=s.reshape(N))
    if fmt.startswith("w8g") and fmt in GROUPED:
        q, s = quantize_w8(W, GROUPED[fmt])
        return dict(fmt=fmt, K=K, N=N, qweight=q, scales=s)
    if fmt.startswith("w4g") and fmt in GROUPED:
        if N % 8:
            raise ValueError("W4 needs N % 8 == 0 (zeros are packed 8 per word along N)")
        q, s16, z = quantize_w4g128(W) if fmt == "w4g128" else quantize_w4(W, GROUPED[fmt])
        return dict(fmt=fmt, K=K, N=N, qweight=_pack_nibbles_rows(q), scales=s16,
                    zeros=_pack_nibbles_rows(np.ascontiguousarray(z.T)))
    if fmt == W4PC:
        if N % 8 or K % 8:
            raise ValueError("W4 needs N % 8 == 0 and K % 8 == 0 (8 codes or zeros per word)")
        q, s16, z = quantize_w4(W, None)
        return dict(fmt=fmt, K=K, N=N, qweight=_pack_nibbles_rows(q), scales=s16.reshape(N),
                    zeros=_pack_nibbles_rows(np.ascontiguousarray(z.T)).reshape(N // 8))
    raise ValueError(f"unknown format {fmt!r}")


def unpack_w4g(P: dict):
    """Canonical grouped W4 words -> (q [N, K] uint8, s fp16 [N, K/G], z [N, K/G] uint8)."""
    q = _unpack_nibbles_rows(P["qweight"])
    z = np.ascontiguousarray(_unpack_nibbles_rows(P["zeros"]).T)
    return q, P["scales"], z


unpack_w4g128 = unpack_w4g


def unpack_w4pc(P: dict):
    """Canonical per-channel W4 words -> (q [N, K] uint8, s fp16 [N], z [N] uint8)."""
    q = _unpack_nibbles_rows(P["qweight"])
    z = _unpack_nibbles_rows(np.asarray(P["zeros"]).reshape(1, -1)).reshape(-1)
    return q, P["scales"], z


def packed_sizes(fmt: str, K: int, N: int):
    """Bytes of (qweight, scales, zeros) in the canonical layout."""
    if fmt == "w8pc":
        return K * N, 2 * N, 0
    if fmt.startswith("w8g") and fmt in GROUPED:
        return K * N, 2 * N * (K // GROUPED[fmt]), 0
    if fmt.startswith("w4g") and fmt in GROUPED:
        G = GROUPED[fmt]
        return K * N // 2, 2 * N * (K // G), (K // G) * (N // 8) * 4
    if fmt == W4PC:
        return K * N // 2, 2 * N, (N // 8) * 4
    raise ValueError(fmt)


# ---------------------------------------------------------------- dequantise
def dequant(P: dict, rows=None) -> np.ndarray:
    """Exact fp32 dequantised weight Wd[N, K] (or only the given output rows)."""
    fmt, K = P["fmt"], P["K"]
    sel = slice(None) if rows is None else np.asarray(rows)
    if fmt == "w8pc" or (fmt.startswith("w8g") and fmt in GROUPED):
        q = P["qweight"][sel].astype(np.float32)
        s = bf16_bits_to_f32(P["scales"][sel])
        if fmt == "w8pc":
            return q * s[:, None]
        n, G = q.shape[0], GROUPED[fmt]
        return (q.reshape(n, K // G, G) * s[:, :, None]).reshape(n, K)
    if fmt.startswith("w4g") and fmt in GROUPED:
        q, s16, z = unpack_w4g(dict(qweight=P["qweight"][sel], scales=P["scales"][sel], zeros=P["zeros"]))
        if rows is not None:
            z = z[np.asarray(rows)]
        n, G = q.shape[0], GROUPED[fmt]
        d = q.astype(np.float32).reshape(n, K // G, G) - z.astype(np.float32)[:, :, None]
        return (d * s16.astype(np.float32)[:, :, None]).reshape(n, K)
    if fmt == W4PC:
        q, s16, z = unpack_w4pc(dict(qweight=P["qweight"][sel], scales=P["scales"][sel], zeros=P["zeros"]))
        if rows is not None:
            z = z[np.asarray(rows)]
        d = q.astype(np.float32) - z.astype(np.float32)[:, None]
        return d * s16.astype(np.float32)[:, None]
    raise ValueError(fmt)
