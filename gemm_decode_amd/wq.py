"""Python binding of libwq.so (the C ABI in include/wq.h), loaded with ctypes.

Argument marshalling only: every computation runs in the library's HIP kernels.
PyTorch supplies device memory (tensors) and streams; the functions below have
the names of the C entry points declared in include/wq.h and take tensors where
the C functions take device pointers.

Importing this package fails loudly (ImportError) when libwq.so has not been
built; there is no fallback implementation.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

__all__ = [
    "FMT", "CANONICAL", "GFX950", "WqError", "PackedWeight", "lib",
    "wq_abi_version", "wq_status_string", "wq_last_error", "wq_packed_sizes", "wq_dispatch_kind",
    "wq_gemv_max_waves", "wq_gemv_max_split",
    "wq_pack", "wq_pack_bf16", "wq_repack", "wq_unrepack", "wq_workspace_size", "wq_gemv", "wq_gemv_ex", "wq_gemm", "wq_linear",
    "wq_lm_head_topk_workspace_size", "wq_lm_head_topk",
    "wq_linear_perm_workspace_size", "wq_linear_perm", "wq_linear_static", "STATIC_SCRATCH_BYTES",
    "wq_moe_linear", "quantize_experts", "EPILOGUE_NONE", "EPILOGUE_SILU_MUL",
    "ACT", "wq_linear_act", "wq_gemv_act", "wq_gemm_act", "wq_linear_residual", "wq_gemv_residual",
    "wq_gemm_residual",
    "wq_tune_pick", "wq_tune", "wq_tune_cache_set", "wq_tune_cache_get", "wq_tune_cache_clear",
    "wq_tune_cache_save", "wq_tune_cache_load", "quantize", "workspace",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libwq.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python -m gemm_decode_amd.build` "
                      "(or __graft_entry__.build()) first")
lib = C.CDLL(LIB_PATH)

FMT = {"w8pc": 0, "w8g128": 1, "w4g128": 2, "w4pc": 3, "w8g32": 4, "w8g64": 5, "w4g32": 6, "w4g64": 7}
FMT_NAME = {v: k for k, v in FMT.items()}
CANONICAL, GFX950 = 0, 1
KIND_GEMV, KIND_GEMM = 0, 1
GEMM_TILES = 28
MMA_TILES = range(20, 24)              # GEMM tiles of the matrix-core GEMV kernel (M <= 16)
TUNE_LAT_SLOTS = 28                      # WQ_TUNE_LAT_SLOTS: entries wq_tune writes to lat_us
SPLIT_GRID = (1, 2, 4, 8, 16, 32)
WAVES_GRID = (1, 2, 4, 8, 16)
ROWS_GRID = (4, 8, 16)
GEMV_PREFETCH = 0x100                    # WQ_GEMV_PREFETCH: rows flag, slice prefetch
GEMV_MFMA = 0x200                        # WQ_GEMV_MFMA: rows flag: the matrix-core GEMV (rows = 16 NB)
STATIC_SCRATCH_BYTES = 64 << 20          # WQ_STATIC_SCRATCH_BYTES: the scratch of wq_linear_static
EPILOGUE_NONE, EPILOGUE_SILU_MUL = 0, 1  # WQ_EPILOGUE_*: epilogues of wq_moe_linear
ACT = {"bf16": 0, "f16": 1}              # WQ_ACT_*: activation types of the *_act entry points


def gemv_cache_value(split_k: int, waves: int = 0, rows: int = 0) -> int:
    """Tuner-cache encoding of a GEMV choice (split_k | waves << 8 | rows << 16)."""
    return split_k | (waves << 8) | (rows << 16)


class WqWeightC(C.Structure):
    _fields_ = [("fmt", C.c_int32), ("layout", C.c_int32), ("K", C.c_int64), ("N", C.c_int64),
                ("qweight", C.c_void_p), ("scales", C.c_void_p), ("zeros", C.c_void_p)]


_P = C.POINTER
_W = _P(WqWeightC)
_SIGS = {
    "wq_abi_version": (C.c_int, []),
    "wq_status_string": (C.c_char_p, [C.c_int]),
    "wq_last_error": (C.c_char_p, []),
    "wq_packed_sizes": (C.c_int, [C.c_int, C.c_int, C.c_int64, C.c_int64, _P(C.c_size_t), _P(C.c_size_t), _P(C.c_size_t)]),
    "wq_dispatch_kind": (C.c_int, [C.c_int64]),
    "wq_gemv_max_waves": (C.c_int, [C.c_int, C.c_int64, C.c_int]),
    "wq_gemv_max_split": (C.c_int, [C.c_int, C.c_int64]),
    "wq_pack": (C.c_int, [C.c_void_p, _W, C.c_void_p]),
    "wq_pack_bf16": (C.c_int, [C.c_void_p, _W, C.c_void_p]),
    "wq_repack": (C.c_int, [_W, _W, C.c_void_p]),
    "wq_unrepack": (C.c_int, [_W, _W, C.c_void_p]),
    "wq_workspace_size": (C.c_int, [_W, C.c_int64, _P(C.c_size_t)]),
    "wq_gemv": (C.c_int, [_W, C.c_void_p, C.c_int64, C.c_void_p, C.c_int, C.c_void_p, C.c_size_t, C.c_void_p]),
    "wq_gemv_ex": (C.c_int, [_W, C.c_void_p, C.c_int64, C.c_void_p, C.c_int, C.c_int, C.c_int, C.c_void_p, C.c_size_t, C.c_void_p]),
    "wq_gemm": (C.c_int, [_W, C.c_void_p, C.c_int64, C.c_void_p, C.c_int, C.c_void_p, C.c_size_t, C.c_void_p]),
    "wq_linear": (C.c_int, [_W, C.c_void_p, C.c_int64, C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]),
    "wq_linear_static": (C.c_int, [_W, C.c_void_p, C.c_int64, C.c_void_p, C.c_void_p]),
    "wq_linear_act": (C.c_int, [_W, C.c_int, C.c_void_p, C.c_int64, C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]),
    "wq_gemv_act": (C.c_int, [_W, C.c_int, C.c_void_p, C.c_int64, C.c_void_p, C.c_int, C.c_int, C.c_int, C.c_void_p,
                              C.c_size_t, C.c_void_p]),
    "wq_gemm_act": (C.c_int, [_W, C.c_int, C.c_void_p, C.c_int64, C.c_void_p, C.c_int, C.c_void_p, C.c_size_t,
                              C.c_void_p]),
    "wq_linear_residual": (C.c_int, [_W, C.c_int, C.c_void_p, C.c_int64, C.c_void_p, C.c_void_p, C.c_void_p,
                                     C.c_size_t, C.c_void_p]),
    "wq_gemv_residual": (C.c_int, [_W, C.c_int, C.c_void_p, C.c_int64, C.c_void_p, C.c_void_p, C.c_int, C.c_int,
                                   C.c_int, C.c_void_p, C.c_size_t, C.c_void_p]),
    "wq_gemm_residual": (C.c_int, [_W, C.c_int, C.c_void_p, C.c_int64, C.c_void_p, C.c_void_p, C.c_int, C.c_void_p,
                                   C.c_size_t, C.c_void_p]),
    "wq_moe_linear": (C.c_int, [_W, C.c_int, C.c_void_p, C.c_void_p, C.c_int64, C.c_void_p, C.c_int, C.c_void_p]),
    "wq_lm_head_topk_workspace_size": (C.c_int, [_W, C.c_int64, C.c_int, _P(C.c_size_t)]),
    "wq_linear_perm_workspace_size": (C.c_int, [_W, C.c_int64, _P(C.c_size_t)]),
    "wq_linear_perm": (C.c_int, [_W, C.c_void_p, C.c_void_p, C.c_int64, C.c_void_p, C.c_void_p, C.c_size_t,
                                 C.c_void_p]),
    "wq_lm_head_topk": (C.c_int, [_W, C.c_void_p, C.c_int64, C.c_int, C.c_float, C.c_void_p, C.c_void_p,
                                  C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]),
    "wq_tune_pick": (C.c_int, [_P(C.c_double), C.c_int]),
    "wq_tune": (C.c_int, [_W, C.c_int, C.c_int64, C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t,
                          C.c_int, C.c_int, C.c_void_p, _P(C.c_int), _P(C.c_double)]),
    "wq_tune_cache_set": (C.c_int, [C.c_char_p, C.c_int, C.c_int64, C.c_int64, C.c_int64, C.c_int, C.c_int]),
    "wq_tune_cache_get": (C.c_int, [C.c_char_p, C.c_int, C.c_int64, C.c_int64, C.c_int64, C.c_int, _P(C.c_int)]),
    "wq_tune_cache_clear": (C.c_int, []),
    "wq_tune_cache_save": (C.c_int, [C.c_char_p]),
    "wq_tune_cache_load": (C.c_int, [C.c_char_p]),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(lib, _name)
    _f.restype, _f.argtypes = _res, _args


class WqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {wq_status_string(status)} ({wq_last_error()})")


def _check(st: int, where: str) -> None:
    if st != 0:
        raise WqError(st, where)


def _stream(stream) -> C.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _ptr(t) -> C.c_void_p:
    return C.c_void_p(0 if t is None else t.data_ptr())


# ------------------------------------------------------------------ host info
def wq_abi_version() -> int:
    return lib.wq_abi_version()


def wq_status_string(st: int) -> str:
    return lib.wq_status_string(st).decode()


def wq_last_error() -> str:
    return lib.wq_last_error().decode()


def wq_packed_sizes(fmt, layout: int, K: int, N: int):
    q, s, z = C.c_size_t(), C.c_size_t(), C.c_size_t()
    _check(lib.wq_packed_sizes(_fmt(fmt), layout, K, N, C.byref(q), C.byref(s), C.byref(z)),
           "wq_packed_sizes")
    return q.value, s.value, z.value


def wq_dispatch_kind(M: int) -> int:
    return lib.wq_dispatch_kind(M)


def wq_gemv_max_waves(fmt, M: int, rows: int = 16) -> int:
    return lib.wq_gemv_max_waves(_fmt(fmt), M, rows)


def wq_gemv_max_split(fmt, K: int) -> int:
    return lib.wq_gemv_max_split(_fmt(fmt), K)


def _fmt(fmt) -> int:
    return FMT[fmt] if isinstance(fmt, str) else int(fmt)


# ------------------------------------------------------------- packed weights
class PackedWeight:
    """Device buffers of one packed weight (owned by torch tensors) plus its
    descriptor.  ``qweight``/``scales``/``zeros`` are flat uint8 tensors."""

    def __init__(self, fmt, layout: int, K: int, N: int, device="cuda", experts: int = 1):
        self.fmt, self.layout, self.K, self.N, self.experts = _fmt(fmt), layout, K, N, experts
        qb, sb, zb = wq_packed_sizes(self.fmt, layout, K, N)
        self.qweight = torch.empty(qb * experts, dtype=torch.uint8, device=device)
        self.scales = torch.empty(sb * experts, dtype=torch.uint8, device=device)
        self.zeros = torch.empty(zb * experts, dtype=torch.uint8, device=device) if zb else None

    def expert(self, e: int) -> "PackedWeight":
        """A view of expert e of a stacked weight (its own qweight / scales / zeros)."""
        qb, sb, zb = wq_packed_sizes(self.fmt, self.layout, self.K, self.N)
        v = PackedWeight.__new__(PackedWeight)
        v.fmt, v.layout, v.K, v.N, v.experts = self.fmt, self.layout, self.K, self.N, 1
        v.qweight = self.qweight[e * qb:(e + 1) * qb]
        v.scales = self.scales[e * sb:(e + 1) * sb]
        v.zeros = None if self.zeros is None else self.zeros[e * zb:(e + 1) * zb]
        return v

    @property
    def fmt_name(self) -> str:
        return FMT_NAME[self.fmt]

    def desc(self) -> WqWeightC:
        return WqWeightC(self.fmt, self.layout, self.K, self.N, self.qweight.data_ptr(),
                         self.scales.data_ptr(), 0 if self.zeros is None else self.zeros.data_ptr())

    def nbytes(self) -> int:
        return self.qweight.numel() + self.scales.numel() + (0 if self.zeros is None else self.zeros.numel())

    def clone(self) -> "PackedWeight":
        c = PackedWeight.__new__(PackedWeight)
        c.fmt, c.layout, c.K, c.N, c.experts = self.fmt, self.layout, self.K, self.N, self.experts
        c.qweight, c.scales = self.qweight.clone(), self.scales.clone()
        c.zeros = None if self.zeros is None else self.zeros.clone()
        return c


def wq_pack(w: torch.Tensor, out: PackedWeight, stream=None) -> None:
    assert w.dtype == torch.float32 and w.is_contiguous() and tuple(w.shape) == (out.N, out.K)
    d = out.desc()
    _check(lib.wq_pack(_ptr(w), C.byref(d), _stream(stream)), "wq_pack")


def wq_pack_bf16(w: torch.Tensor, out: PackedWeight, stream=None) -> None:
    assert w.dtype == torch.bfloat16 and w.is_contiguous() and tuple(w.shape) == (out.N, out.K)
    d = out.desc()
    _check(lib.wq_pack_bf16(_ptr(w), C.byref(d), _stream(stream)), "wq_pack_bf16")


def wq_repack(src: PackedWeight, dst: PackedWeight, stream=None) -> None:
    a, b = src.desc(), dst.desc()
    _check(lib.wq_repack(C.byref(a), C.byref(b), _stream(stream)), "wq_repack")


def wq_unrepack(src: PackedWeight, dst: PackedWeight, stream=None) -> None:
    a, b = src.desc(), dst.desc()
    _check(lib.wq_unrepack(C.byref(a), C.byref(b), _stream(stream)), "wq_unrepack")


def quantize(w: torch.Tensor, fmt, stream=None, keep_canonical: bool = False):
    """wq_pack (fp32 w) or wq_pack_bf16 (bf16 w) into the canonical layout, then
    wq_repack into the gfx950 layout."""
    N, K = w.shape
    can = PackedWeight(fmt, CANONICAL, K, N, device=w.device)
    (wq_pack_bf16 if w.dtype == torch.bfloat16 else wq_pack)(w, can, stream)
    g = PackedWeight(fmt, GFX950, K, N, device=w.device)
    wq_repack(can, g, stream)
    return (g, can) if keep_canonical else g


def quantize_experts(ws, fmt, stream=None) -> PackedWeight:
    """Pack E weights of one shape (a sequence of [N][K] fp32 or bf16 tensors) into one
    stacked gfx950 weight for wq_moe_linear: expert e is wq_pack + wq_repack of ws[e]."""
    N, K = ws[0].shape
    out = PackedWeight(fmt, GFX950, K, N, device=ws[0].device, experts=len(ws))
    for e, w in enumerate(ws):
        can = PackedWeight(fmt, CANONICAL, K, N, device=w.device)
        (wq_pack_bf16 if w.dtype == torch.bfloat16 else wq_pack)(w, can, stream)
        wq_repack(can, out.expert(e), stream)
    return out


# ---------------------------------------------------------------- the linear
def wq_workspace_size(w: PackedWeight, M: int) -> int:
    d, n = w.desc(), C.c_size_t()
    _check(lib.wq_workspace_size(C.byref(d), M, C.byref(n)), "wq_workspace_size")
    return n.value


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A workspace buffer (scratch for split-K partial sums; needs no initialisation)."""
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def _xy(x: torch.Tensor, y: torch.Tensor, w: PackedWeight, dtype=None):
    dtype = torch.bfloat16 if dtype is None else dtype
    assert x.dtype == dtype and y.dtype == dtype
    assert x.is_contiguous() and y.is_contiguous()
    M = x.numel() // w.K
    assert x.numel() == M * w.K and y.numel() == M * w.N, "x/y sizes do not match the weight"
    return M


def wq_gemv(w: PackedWeight, x: torch.Tensor, y: torch.Tensor, split_k: int = 0,
            ws: torch.Tensor | None = None, stream=None) -> None:
    M, d = _xy(x, y, w), w.desc()
    _check(lib.wq_gemv(C.byref(d), _ptr(x), M, _ptr(y), split_k, _ptr(ws),
                       0 if ws is None else ws.numel(), _stream(stream)), "wq_gemv")


def wq_gemv_ex(w: PackedWeight, x: torch.Tensor, y: torch.Tensor, split_k: int, waves: int = 0,
               rows: int = 0, ws: torch.Tensor | None = None, stream=None) -> None:
    M, d = _xy(x, y, w), w.desc()
    _check(lib.wq_gemv_ex(C.byref(d), _ptr(x), M, _ptr(y), split_k, waves, rows, _ptr(ws),
                          0 if ws is None else ws.numel(), _stream(stream)), "wq_gemv_ex")


def wq_gemm(w: PackedWeight, x: torch.Tensor, y: torch.Tensor, tile: int = 0,
            ws: torch.Tensor | None = None, stream=None) -> None:
    M, d = _xy(x, y, w), w.desc()
    _check(lib.wq_gemm(C.byref(d), _ptr(x), M, _ptr(y), tile, _ptr(ws),
                       0 if ws is None else ws.numel(), _stream(stream)), "wq_gemm")


def wq_linear(w: PackedWeight, x: torch.Tensor, y: torch.Tensor, ws: torch.Tensor | None = None,
              stream=None) -> None:
    M, d = _xy(x, y, w), w.desc()
    _check(lib.wq_linear(C.byref(d), _ptr(x), M, _ptr(y), _ptr(ws),
                         0 if ws is None else ws.numel(), _stream(stream)), "wq_linear")


def _act(x: torch.Tensor) -> int:
    """Activation type of a bf16 or fp16 tensor."""
    return ACT["f16"] if x.dtype == torch.float16 else ACT["bf16"]


def wq_linear_act(w: PackedWeight, x: torch.Tensor, y: torch.Tensor, ws: torch.Tensor | None = None,
                  stream=None) -> None:
    """wq_linear for bf16 or fp16 x and y (the activation type follows x)."""
    M, d = _xy(x, y, w, x.dtype), w.desc()
    _check(lib.wq_linear_act(C.byref(d), _act(x), _ptr(x), M, _ptr(y), _ptr(ws),
                             0 if ws is None else ws.numel(), _stream(stream)), "wq_linear_act")


def wq_gemv_act(w: PackedWeight, x: torch.Tensor, y: torch.Tensor, split_k: int = 0, waves: int = 0,
                rows: int = 0, ws: torch.Tensor | None = None, stream=None) -> None:
    M, d = _xy(x, y, w, x.dtype), w.desc()
    _check(lib.wq_gemv_act(C.byref(d), _act(x), _ptr(x), M, _ptr(y), split_k, waves, rows, _ptr(ws),
                           0 if ws is None else ws.numel(), _stream(stream)), "wq_gemv_act")


def wq_gemm_act(w: PackedWeight, x: torch.Tensor, y: torch.Tensor, tile: int = 0,
                ws: torch.Tensor | None = None, stream=None) -> None:
    M, d = _xy(x, y, w, x.dtype), w.desc()
    _check(lib.wq_gemm_act(C.byref(d), _act(x), _ptr(x), M, _ptr(y), tile, _ptr(ws),
                           0 if ws is None else ws.numel(), _stream(stream)), "wq_gemm_act")


def _res(r: torch.Tensor, y: torch.Tensor):
    assert r.dtype == y.dtype and r.is_contiguous() and r.numel() == y.numel(), "residual must match y"
    return _ptr(r)


def wq_linear_residual(w: PackedWeight, x: torch.Tensor, r: torch.Tensor, y: torch.Tensor,
                       ws: torch.Tensor | None = None, stream=None) -> None:
    """y = x . dequant(W)^T + r, rounded once (r may be y itself); bf16 or fp16 as x."""
    M, d = _xy(x, y, w, x.dtype), w.desc()
    _check(lib.wq_linear_residual(C.byref(d), _act(x), _ptr(x), M, _res(r, y), _ptr(y), _ptr(ws),
                                  0 if ws is None else ws.numel(), _stream(stream)), "wq_linear_residual")


def wq_gemv_residual(w: PackedWeight, x: torch.Tensor, r: torch.Tensor, y: torch.Tensor, split_k: int = 0,
                     waves: int = 0, rows: int = 0, ws: torch.Tensor | None = None, stream=None) -> None:
    M, d = _xy(x, y, w, x.dtype), w.desc()
    _check(lib.wq_gemv_residual(C.byref(d), _act(x), _ptr(x), M, _res(r, y), _ptr(y), split_k, waves, rows,
                                _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)), "wq_gemv_residual")


def wq_gemm_residual(w: PackedWeight, x: torch.Tensor, r: torch.Tensor, y: torch.Tensor, tile: int = 0,
                     ws: torch.Tensor | None = None, stream=None) -> None:
    M, d = _xy(x, y, w, x.dtype), w.desc()
    _check(lib.wq_gemm_residual(C.byref(d), _act(x), _ptr(x), M, _res(r, y), _ptr(y), tile, _ptr(ws),
                                0 if ws is None else ws.numel(), _stream(stream)), "wq_gemm_residual")


def wq_linear_static(w: PackedWeight, x: torch.Tensor, y: torch.Tensor, stream=None) -> None:
    """wq_linear with the library's static scratch instead of a workspace (no allocation)."""
    M, d = _xy(x, y, w), w.desc()
    _check(lib.wq_linear_static(C.byref(d), _ptr(x), M, _ptr(y), _stream(stream)), "wq_linear_static")


def wq_moe_linear(w: PackedWeight, x: torch.Tensor, offsets: torch.Tensor, y: torch.Tensor,
                  epilogue: int = EPILOGUE_NONE, stream=None) -> None:
    """x bf16 [T][K] grouped by expert, offsets int32 [E + 1] (device), y bf16 [T][N] (or
    [T][N / 2] with the gated epilogue); w a stacked weight of E experts."""
    assert x.dtype == torch.bfloat16 and x.is_contiguous() and y.dtype == torch.bfloat16 and y.is_contiguous()
    assert offsets.dtype == torch.int32 and offsets.is_contiguous() and offsets.numel() == w.experts + 1
    T = x.numel() // w.K
    assert x.numel() == T * w.K
    assert y.numel() == T * (w.N // 2 if epilogue == EPILOGUE_SILU_MUL else w.N)
    d = w.desc()
    _check(lib.wq_moe_linear(C.byref(d), w.experts, _ptr(x), _ptr(offsets), T, _ptr(y), epilogue,
                             _stream(stream)), "wq_moe_linear")


# ------------------------------------------------------------ LM head + top-k
def wq_lm_head_topk_workspace_size(w: PackedWeight, M: int, k: int) -> int:
    d, n = w.desc(), C.c_size_t()
    _check(lib.wq_lm_head_topk_workspace_size(C.byref(d), M, k, C.byref(n)), "wq_lm_head_topk_workspace_size")
    return n.value


def wq_lm_head_topk(w: PackedWeight, x: torch.Tensor, k: int, temperature: float, u: torch.Tensor,
                    top_vals: torch.Tensor, top_idx: torch.Tensor, tokens: torch.Tensor,
                    ws: torch.Tensor, stream=None) -> None:
    """x bf16 [M][K]; u fp32 [M]; outputs top_vals bf16 [M][k], top_idx int32 [M][k],
    tokens int32 [M] (all on the device)."""
    assert x.dtype == torch.bfloat16 and x.is_contiguous()
    M = x.numel() // w.K
    assert x.numel() == M * w.K
    assert u.dtype == torch.float32 and u.numel() == M
    assert top_vals.dtype == torch.bfloat16 and top_vals.numel() == M * k
    assert top_idx.dtype == torch.int32 and top_idx.numel() == M * k
    assert tokens.dtype == torch.int32 and tokens.numel() == M
    d = w.desc()
    _check(lib.wq_lm_head_topk(C.byref(d), _ptr(x), M, k, float(temperature), _ptr(u), _ptr(top_vals),
                               _ptr(top_idx), _ptr(tokens), _ptr(ws), 0 if ws is None else ws.numel(),
                               _stream(stream)), "wq_lm_head_topk")


def wq_linear_perm_workspace_size(w: PackedWeight, M: int) -> int:
    d, n = w.desc(), C.c_size_t()
    _check(lib.wq_linear_perm_workspace_size(C.byref(d), M, C.byref(n)), "wq_linear_perm_workspace_size")
    return n.value


def wq_linear_perm(w: PackedWeight, x: torch.Tensor, perm: torch.Tensor, y: torch.Tensor,
                   ws: torch.Tensor, stream=None) -> None:
    """x bf16 [M][K], perm int32 [K], y bf16 [M][N] (all on the device): y = x[:, perm]
    times the stored weight."""
    M = _xy(x, y, w)
    assert perm.dtype == torch.int32 and perm.is_contiguous() and perm.numel() == w.K
    d = w.desc()
    _check(lib.wq_linear_perm(C.byref(d), _ptr(x), _ptr(perm), M, _ptr(y), _ptr(ws),
                              0 if ws is None else ws.numel(), _stream(stream)), "wq_linear_perm")


# ---------------------------------------------------------------------- tuner
def wq_tune_pick(lat) -> int:
    arr = (C.c_double * len(lat))(*lat)
    return lib.wq_tune_pick(arr, len(lat))


def wq_tune(copies, x: torch.Tensor, y: torch.Tensor, ws: torch.Tensor | None = None,
            warmup: int = 1000, iters: int = 1000, stream=None):
    """Returns (chosen split_k or tile, mean microseconds per split_k (best waves) or tile)."""
    M = _xy(x, y, copies[0])
    arr = (WqWeightC * len(copies))(*[c.desc() for c in copies])
    chosen = C.c_int()
    lat = (C.c_double * TUNE_LAT_SLOTS)(*([-1.0] * TUNE_LAT_SLOTS))
    _check(lib.wq_tune(arr, len(copies), M, _ptr(x), _ptr(y), _ptr(ws), 0 if ws is None else ws.numel(),
                       warmup, iters, _stream(stream), C.byref(chosen), lat), "wq_tune")
    n = len(SPLIT_GRID) if wq_dispatch_kind(M) == KIND_GEMV else GEMM_TILES
    return chosen.value, list(lat)[:n]


def wq_tune_cache_set(fmt, K: int, N: int, M: int, kind: int, value: int, device_tag: str = "") -> None:
    _check(lib.wq_tune_cache_set(device_tag.encode(), _fmt(fmt), K, N, M, kind, value), "wq_tune_cache_set")


def wq_tune_cache_get(fmt, K: int, N: int, M: int, kind: int, device_tag: str = ""):
    v = C.c_int()
    st = lib.wq_tune_cache_get(device_tag.encode(), _fmt(fmt), K, N, M, kind, C.byref(v))
    return v.value if st == 0 else None


def wq_tune_cache_clear() -> None:
    _check(lib.wq_tune_cache_clear(), "wq_tune_cache_clear")


def wq_tune_cache_save(path: str) -> None:
    _check(lib.wq_tune_cache_save(os.fsencode(path)), "wq_tune_cache_save")


def wq_tune_cache_load(path: str) -> None:
    _check(lib.wq_tune_cache_load(os.fsencode(path)), "wq_tune_cache_load")
