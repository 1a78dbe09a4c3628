"""GPU: fp16 activations (wq_linear_act / wq_gemv_act / wq_gemm_act with WQ_ACT_F16)
through the C ABI against the oracle's layer on fp16 x (oracle/linear.py, act="f16"):
every GEMV split and dot2 launch shape, every GEMM tile id, one-hot rows exact (y =
fp16 of the dequantised weight), fp16 x at the ends of its range (subnormal and near
65504), the tuned launch of the bf16 layer taken over, the full (5120, 27648) shape, and
the bf16 activation type through the same entry points bit-identical to the plain ones.
Needs an MI355X."""
import numpy as np
import pytest
import torch

import oracle.linear as OL
import oracle.quant as OQ
import synth
from gpu_util import DEV, bf16_bits, quantize_on_gpu, sample_rows, to_dev_bf16

pytestmark = pytest.mark.gpu
FMTS = ["w8pc", "w8g128", "w4g128", "w4pc", "w4g32", "w8g64"]


@pytest.fixture(scope="module")
def wq(wqlib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return wqlib


def _dev16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.float16)


def _y16(wq, g, x_bits, call):
    M = x_bits.shape[0]
    y = torch.empty((M, g.N), dtype=torch.float16, device=DEV)
    call(_dev16(x_bits), y)
    torch.cuda.synchronize()
    return y.view(torch.int16).cpu().numpy().view(np.uint16)


def _parity16(y_bits, y_ref, what):
    st = OL.compare(y_bits, y_ref, act="f16")
    assert st["fails"] == 0, f"{what}: {st}"
    # exact products and fp32 sums: what remains is the fp16 rounding of y (2^-11 relative)
    assert st["max_ratio"] < 0.1, f"{what}: error beyond fp16 output rounding: {st}"
    return st


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("K,N", [(9088, 776), (1024, 264)])
def test_gemv_every_split_and_launch_shape(wq, fmt, K, N):
    W = synth.weight(171, K, N, fmt.startswith("w4"))
    g, _ = quantize_on_gpu(wq, W, fmt)
    P = OQ.pack(fmt, W)
    for M in (1, 3, 7):
        x = synth.activation_f16(171, K, M)
        y_ref = OL.ref_linear(x, P, act="f16")
        ws = wq.workspace(wq.wq_workspace_size(g, M))
        smax = wq.wq_gemv_max_split(fmt, K)
        for split in [s for s in (1, 2, 4, 8, 32) if s <= smax]:
            _parity16(_y16(wq, g, x, lambda xd, y: wq.wq_gemv_act(g, xd, y, split, ws=ws)), y_ref,
                      f"{fmt} gemv K={K} M={M} split={split}")
        for rows in (4, 8, 16):
            cap = wq.wq_gemv_max_waves(fmt, M, rows)
            for waves in sorted({1, cap}):
                _parity16(_y16(wq, g, x, lambda xd, y: wq.wq_gemv_act(g, xd, y, 1, waves, rows, ws=ws)), y_ref,
                          f"{fmt} gemv K={K} M={M} rows={rows} waves={waves}")
        for rows in (16 | wq.GEMV_MFMA, 8 | wq.GEMV_PREFETCH):
            if wq.wq_gemv_max_waves(fmt, M, rows) < 1:
                continue
            with pytest.raises(wq.WqError) as e:
                _y16(wq, g, x, lambda xd, y: wq.wq_gemv_act(g, xd, y, 1, 1, rows, ws=ws))
            assert e.value.status == 2


@pytest.mark.parametrize("fmt", FMTS)
def test_gemm_every_tile(wq, fmt):
    K, N = 1024, 520
    W = synth.weight(172, K, N, fmt.startswith("w4"))
    g, _ = quantize_on_gpu(wq, W, fmt)
    P = OQ.pack(fmt, W)
    for M in (8, 13, 40, 300):
        x = synth.activation_f16(172, K, M)
        y_ref = OL.ref_linear(x, P, act="f16")
        ws = wq.workspace(wq.wq_workspace_size(g, M))
        for tile in range(1, wq.GEMM_TILES + 1):
            _parity16(_y16(wq, g, x, lambda xd, y: wq.wq_gemm_act(g, xd, y, tile=tile, ws=ws)), y_ref,
                      f"{fmt} gemm M={M} tile={tile}")
        _parity16(_y16(wq, g, x, lambda xd, y: wq.wq_linear_act(g, xd, y, ws=ws)), y_ref, f"{fmt} linear M={M}")
        _parity16(_y16(wq, g, x, lambda xd, y: wq.wq_gemm_act(g, xd, y, tile=9, ws=None)), y_ref,
                  f"{fmt} gemm M={M} tile 9 without workspace")


@pytest.mark.parametrize("fmt", FMTS)
def test_one_hot_is_exact(wq, fmt):
    """x = e_k gives fp16 of the exact dequantised weight on every path."""
    K, N = 1024, 264
    W = synth.weight(173, K, N, fmt.startswith("w4"))
    g, _ = quantize_on_gpu(wq, W, fmt)
    deq = OQ.dequant(OQ.pack(fmt, W)).T.copy()                    # [K][N] fp32, exact
    edges = [0, 31, 32, 63, 64, 127, 128, 511, 512, K - 1]
    for M, ks in ((3, edges[:3]), (7, edges[3:10]), (10, edges)):
        x = np.zeros((M, K), dtype=np.uint16)
        for m, k in enumerate(ks):
            x[m, k] = 0x3C00                                      # fp16 1.0
        want = deq[ks].astype(np.float16).view(np.uint16)         # nearest even
        ws = wq.workspace(wq.wq_workspace_size(g, M))
        if M < 8:
            for rows in (4, 8, 16):
                got = _y16(wq, g, x, lambda xd, y: wq.wq_gemv_act(g, xd, y, 1, 0, rows, ws=None))
                assert np.array_equal(got, want), f"{fmt} gemv rows={rows}"
        else:
            for tile in range(1, wq.GEMM_TILES + 1):
                got = _y16(wq, g, x, lambda xd, y: wq.wq_gemm_act(g, xd, y, tile=tile, ws=ws))
                assert np.array_equal(got, want), f"{fmt} gemm tile={tile}"


@pytest.mark.parametrize("fmt", ["w8pc", "w4g128", "w4g32"])
def test_range_ends(wq, fmt):
    """fp16 x at the ends of its range: subnormals (k 2^-24) with weights scaled up,
    and magnitudes near 65504 with weights scaled down; both exact in fp32 products."""
    K, N = 2048, 264
    rng = np.random.default_rng(174)
    for scale_w, xv in ((2.0 ** 16, rng.integers(-1023, 1024, size=(9, K)).astype(np.float64) * 2.0 ** -24),
                        (2.0 ** -16, rng.uniform(-65504, 65504, size=(9, K)))):
        W = (synth.weight(174, K, N, fmt.startswith("w4")) * np.float32(scale_w)).astype(np.float32)
        g, _ = quantize_on_gpu(wq, W, fmt)
        P = OQ.pack(fmt, W)
        x = xv.astype(np.float16).view(np.uint16)
        for M in (3, 9):
            xm = np.ascontiguousarray(x[:M])
            y_ref = OL.ref_linear(xm, P, act="f16")
            assert np.all(np.abs(y_ref) < 60000)
            ws = wq.workspace(wq.wq_workspace_size(g, M))
            _parity16(_y16(wq, g, xm, lambda xd, y: wq.wq_linear_act(g, xd, y, ws=ws)), y_ref,
                      f"{fmt} scale_w={scale_w} M={M}")
            if M >= 8:
                for tile in (2, 9, 10, 14, 24):
                    _parity16(_y16(wq, g, xm, lambda xd, y: wq.wq_gemm_act(g, xd, y, tile=tile, ws=ws)), y_ref,
                              f"{fmt} scale_w={scale_w} tile={tile}")


@pytest.mark.parametrize("fmt", ["w8pc", "w4g128"])
def test_tuned_launch_taken_over_and_bf16_identity(wq, fmt):
    """A tuned bf16 launch with the matrix-core or prefetch option runs fp16 x on the
    dot2 GEMV; the bf16 activation type through the *_act entry points is bit-identical
    to the plain entry points."""
    K, N, M = 5120, 1024, 4
    W = synth.weight(175, K, N, fmt.startswith("w4"))
    g, _ = quantize_on_gpu(wq, W, fmt)
    P = OQ.pack(fmt, W)
    x16 = synth.activation_f16(175, K, M)
    y_ref = OL.ref_linear(x16, P, act="f16")
    ws = wq.workspace(wq.wq_workspace_size(g, M))
    for rows in (16 | wq.GEMV_MFMA, 4 | wq.GEMV_PREFETCH):
        if wq.wq_gemv_max_waves(fmt, M, rows) < 1:
            continue
        wq.wq_tune_cache_set(fmt, K, N, M, wq.KIND_GEMV, wq.gemv_cache_value(1, 1, rows))
        _parity16(_y16(wq, g, x16, lambda xd, y: wq.wq_linear_act(g, xd, y, ws=ws)), y_ref, f"{fmt} tuned {rows:#x}")
    wq.wq_tune_cache_clear()
    for Mx in (M, 40):
        xb = synth.activation(175, K, Mx)
        ws = wq.workspace(wq.wq_workspace_size(g, Mx))
        ya = torch.empty((Mx, N), dtype=torch.bfloat16, device=DEV)
        yb = torch.empty((Mx, N), dtype=torch.bfloat16, device=DEV)
        wq.wq_linear(g, to_dev_bf16(xb), ya, ws=ws)
        wq.wq_linear_act(g, to_dev_bf16(xb), yb, ws=ws)
        torch.cuda.synchronize()
        assert np.array_equal(bf16_bits(ya), bf16_bits(yb)), f"{fmt} bf16 M={Mx}"


@pytest.mark.parametrize("fmt", ["w8pc", "w4g128"])
def test_full_decode_shape_and_prefill(wq, fmt):
    """(5120, 27648): every output channel at M = 1 and 4, sampled rows at M = 64 and 2048."""
    K, N = 5120, 27648
    W = synth.weight(3, K, N, fmt.startswith("w4"))
    g, _ = quantize_on_gpu(wq, W, fmt)
    P = OQ.pack(fmt, W)
    for M in (1, 4):
        x = synth.activation_f16(3, K, M)
        ws = wq.workspace(wq.wq_workspace_size(g, M))
        _parity16(_y16(wq, g, x, lambda xd, y: wq.wq_linear_act(g, xd, y, ws=ws)), OL.ref_linear(x, P, act="f16"),
                  f"{fmt} M={M}")
    rows = sample_rows(N, 64, seed=3)
    Pr = OQ.pack(fmt, W[rows])
    for M in (64, 2048):
        x = synth.activation_f16(3, K, M)
        ws = wq.workspace(wq.wq_workspace_size(g, M))
        y = _y16(wq, g, x, lambda xd, y: wq.wq_linear_act(g, xd, y, ws=ws))
        _parity16(y[:, rows], OL.ref_linear(x, Pr, act="f16"), f"{fmt} M={M} sampled rows")
