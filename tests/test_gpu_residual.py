"""GPU: the residual epilogue (wq_linear_residual / wq_gemv_residual / wq_gemm_residual)
through the C ABI against the oracle (oracle/linear.py, ref_linear_residual): every GEMV
split and launch option (the matrix-core GEMV included), every GEMM tile id (split-K and
split-tail tiles, whose reductions add the residual), in place (r = y), fp16 activations,
one-hot rows bit-exact, and the full (5120, 27648) shape.  Needs an MI355X."""
import numpy as np
import pytest
import torch

import oracle.linear as OL
import oracle.quant as OQ
import synth
from gpu_util import DEV, bf16_bits, quantize_on_gpu, to_dev_bf16

pytestmark = pytest.mark.gpu
FMTS = ["w8pc", "w8g128", "w4g128", "w4g32"]


@pytest.fixture(scope="module")
def wq(wqlib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return wqlib


def _run(wq, g, x_bits, r_bits, call, inplace=False, f16=False):
    M = x_bits.shape[0]
    dt = torch.float16 if f16 else torch.bfloat16
    xd = torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).to(DEV).view(dt)
    r = torch.from_numpy(np.ascontiguousarray(r_bits).view(np.int16)).to(DEV).view(dt)
    y = r if inplace else torch.empty((M, g.N), dtype=dt, device=DEV)
    call(xd, r, y)
    torch.cuda.synchronize()
    return y.view(torch.int16).cpu().numpy().view(np.uint16)


def _parity(y_bits, ref, what, act="bf16"):
    st = OL.compare(y_bits, ref, act=act)
    assert st["fails"] == 0, f"{what}: {st}"
    assert st["max_ratio"] < (0.6 if act == "bf16" else 0.1), f"{what}: {st}"


def _residual(seed, M, N, f16=False):
    return synth.activation_f16(seed, N, M) if f16 else synth.activation(seed, N, M)


@pytest.mark.parametrize("fmt", FMTS)
def test_gemv_every_split_and_launch_option(wq, fmt):
    K, N = 9088, 776
    W = synth.weight(181, K, N, fmt.startswith("w4"))
    g, _ = quantize_on_gpu(wq, W, fmt)
    P = OQ.pack(fmt, W)
    for M in (1, 3, 7):
        x = synth.activation(181, K, M)
        r = _residual(182, M, N)
        ref = OL.ref_linear_residual(x, P, r)
        ws = wq.workspace(wq.wq_workspace_size(g, M))
        for split in [s for s in (1, 2, 4, 8) if s <= wq.wq_gemv_max_split(fmt, K)]:
            _parity(_run(wq, g, x, r, lambda xd, rd, y: wq.wq_gemv_residual(g, xd, rd, y, split, ws=ws)), ref,
                    f"{fmt} M={M} split={split}")
        for rows in (4, 16, 4 | wq.GEMV_PREFETCH, 16 | wq.GEMV_MFMA, 64 | wq.GEMV_MFMA):
            if wq.wq_gemv_max_waves(fmt, M, rows) < 1:
                continue
            _parity(_run(wq, g, x, r, lambda xd, rd, y: wq.wq_gemv_residual(g, xd, rd, y, 2, 0, rows, ws=ws)), ref,
                    f"{fmt} M={M} rows={rows:#x}")
        _parity(_run(wq, g, x, r, lambda xd, rd, y: wq.wq_linear_residual(g, xd, rd, y, ws=ws), inplace=True), ref,
                f"{fmt} M={M} in place")


@pytest.mark.parametrize("fmt", FMTS)
def test_gemm_every_tile(wq, fmt):
    K, N = 1024, 520
    W = synth.weight(183, K, N, fmt.startswith("w4"))
    g, _ = quantize_on_gpu(wq, W, fmt)
    P = OQ.pack(fmt, W)
    for M in (8, 13, 40, 300):
        x = synth.activation(183, K, M)
        r = _residual(184, M, N)
        ref = OL.ref_linear_residual(x, P, r)
        ws = wq.workspace(wq.wq_workspace_size(g, M))
        for tile in range(1, wq.GEMM_TILES + 1):
            _parity(_run(wq, g, x, r, lambda xd, rd, y: wq.wq_gemm_residual(g, xd, rd, y, tile=tile, ws=ws)), ref,
                    f"{fmt} M={M} tile={tile}")
            _parity(_run(wq, g, x, r, lambda xd, rd, y: wq.wq_gemm_residual(g, xd, rd, y, tile=tile, ws=ws),
                         inplace=True), ref, f"{fmt} M={M} tile={tile} in place")


def test_split_tail_tile(wq):
    """Tile 13 splits a partial last round over K: its reduction adds the residual to the
    tail tiles, the main kernel to the others (M = 2048 on a shape whose tile count exceeds
    the CUs by a partial round)."""
    K, N, M = 1024, 27648, 2048
    for fmt in ("w8pc", "w4g128"):
        W = synth.weight(185, K, N, fmt.startswith("w4"))
        g, _ = quantize_on_gpu(wq, W, fmt)
        rows = np.arange(0, N, 97)
        Pr = OQ.pack(fmt, W[rows]) if fmt == "w8pc" else None
        x = synth.activation(185, K, M)
        r = _residual(186, M, N)
        ws = wq.workspace(wq.wq_workspace_size(g, M))
        y = _run(wq, g, x, r, lambda xd, rd, yy: wq.wq_gemm_residual(g, xd, rd, yy, tile=13, ws=ws), inplace=True)
        if Pr is None:  # W4 rows come in blocks of 8 for the zero-point words
            blocks = np.unique(rows // 8)
            rows = (blocks[:, None] * 8 + np.arange(8)[None, :]).ravel()
            Pr = OQ.pack(fmt, W[rows])
        ref = OL.ref_linear(x, Pr) + OL._x64(r[:, rows])
        _parity(y[:, rows], ref, f"{fmt} tile 13 in place")


@pytest.mark.parametrize("fmt", ["w8pc", "w4g128"])
def test_f16_activations(wq, fmt):
    K, N = 2048, 520
    W = synth.weight(187, K, N, fmt.startswith("w4"))
    g, _ = quantize_on_gpu(wq, W, fmt)
    P = OQ.pack(fmt, W)
    for M in (3, 40):
        x = synth.activation_f16(187, K, M)
        r = _residual(188, M, N, f16=True)
        ref = OL.ref_linear_residual(x, P, r, act="f16")
        ws = wq.workspace(wq.wq_workspace_size(g, M))
        _parity(_run(wq, g, x, r, lambda xd, rd, y: wq.wq_linear_residual(g, xd, rd, y, ws=ws), f16=True), ref,
                f"{fmt} f16 M={M}", act="f16")
        _parity(_run(wq, g, x, r, lambda xd, rd, y: wq.wq_linear_residual(g, xd, rd, y, ws=ws), inplace=True,
                     f16=True), ref, f"{fmt} f16 M={M} in place", act="f16")


@pytest.mark.parametrize("fmt", FMTS)
def test_one_hot_is_exact(wq, fmt):
    """x = e_k: y = bf16(fp32(dequantised weight) + r), one fp32 addition then one rounding."""
    K, N = 1024, 264
    W = synth.weight(189, K, N, fmt.startswith("w4"))
    g, _ = quantize_on_gpu(wq, W, fmt)
    deq = OQ.dequant(OQ.pack(fmt, W)).T.copy()
    for M, ks in ((3, [0, 511, K - 1]), (9, list(range(0, K, 120))[:9])):
        x = synth.one_hot_activation(K, ks)
        r = _residual(190, M, N)
        want = OQ.bf16_rne_bits(deq[ks].astype(np.float32) + OQ.bf16_bits_to_f32(r))
        ws = wq.workspace(wq.wq_workspace_size(g, M))
        got = _run(wq, g, x, r, lambda xd, rd, y: wq.wq_linear_residual(g, xd, rd, y, ws=ws))
        assert np.array_equal(got, want), f"{fmt} M={M}"


def test_full_shape_and_refusals(wq):
    K, N = 5120, 27648
    W = synth.weight(3, K, N, False)
    g, _ = quantize_on_gpu(wq, W, "w8pc")
    P = OQ.pack("w8pc", W)
    x = synth.activation(3, K, 1)
    r = _residual(191, 1, N)
    ws = wq.workspace(wq.wq_workspace_size(g, 1))
    _parity(_run(wq, g, x, r, lambda xd, rd, y: wq.wq_linear_residual(g, xd, rd, y, ws=ws), inplace=True),
            OL.ref_linear_residual(x, P, r), "full shape M=1 in place")
    xd = to_dev_bf16(x)
    y = torch.empty((2, N), dtype=torch.bfloat16, device=DEV)
    d = g.desc()
    import ctypes as C
    L = wq.lib
    # an overlap other than r == y, and a NULL residual, are refused before any launch
    assert L.wq_linear_residual(C.byref(d), 0, wq._ptr(xd), 1, C.c_void_p(y.data_ptr() + 2), wq._ptr(y),
                                None, 0, None) == 1
    assert L.wq_linear_residual(C.byref(d), 0, wq._ptr(xd), 1, None, wq._ptr(y), None, 0, None) == 1
