"""GPU: groups of 32 and 64 (WQ_FMT_W8_G32, W8_G64, W4_G32, W4_G64) through the C ABI
against the oracle (oracle/quant.py, the grouped recipe with G = 32 or 64): bit-exact
packing from fp32 and bf16 weights and the exact inverse of the gfx950 layout, the
GEMV at every split and launch shape it offers, every GEMM tile (those that run as
another tile included), one-hot inputs on both sides of every group edge, the full
(5120, 27648) decode shape with sampled prefill rows, and the no-allocation entry
point.  Needs an MI355X."""
import numpy as np
import pytest
import torch

import oracle.linear as OL
import oracle.quant as OQ
import synth
from gpu_util import (DEV, assert_parity, bf16_bits, canonical_to_host, quantize_on_gpu, sample_rows,
                      to_dev_bf16)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wq(wqlib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return wqlib


def _y(wq, g, x_bits, call):
    M = x_bits.shape[0]
    y = torch.empty((M, g.N), dtype=torch.bfloat16, device=DEV)
    call(to_dev_bf16(x_bits), y)
    torch.cuda.synchronize()
    return bf16_bits(y)


def _keys(fmt):
    return ("qweight", "scales", "zeros") if fmt.startswith("w4") else ("qweight", "scales")


@pytest.mark.parametrize("fmt", OQ.SMALL_GROUPS)
@pytest.mark.parametrize("K,N", [(1024, 264), (640, 40), (128, 8)])
def test_pack_repack_bitexact(wq, fmt, K, N):
    W = synth.weight(160, K, N, fmt.startswith("w4"))
    W[3] = 0                                      # an all-zero row
    W[5, :32] = np.float32(0.5)                   # a constant group: s = 0 (W4) in that group
    g, can = quantize_on_gpu(wq, W, fmt)
    got, want = canonical_to_host(can, fmt), OQ.pack(fmt, W)
    for key in _keys(fmt):
        assert np.array_equal(got[key].view(np.uint8), want[key].view(np.uint8)), key
    Wb = OQ.bf16_rne_bits(W)
    Wt = torch.from_numpy(Wb.view(np.int16)).to(DEV).view(torch.bfloat16)
    gb, canb = wq.quantize(Wt, fmt, keep_canonical=True)
    gotb, wantb = canonical_to_host(canb, fmt), OQ.pack(fmt, OQ.bf16_bits_to_f32(Wb))
    for key in _keys(fmt):
        assert np.array_equal(gotb[key].view(np.uint8), wantb[key].view(np.uint8)), "bf16 " + key
    back = wq.PackedWeight(fmt, wq.CANONICAL, K, N)
    wq.wq_unrepack(g, back)
    torch.cuda.synchronize()
    pairs = [(back.qweight, can.qweight), (back.scales, can.scales)]
    if fmt.startswith("w4"):
        pairs.append((back.zeros, can.zeros))
    for a, b in pairs:
        assert torch.equal(a, b)


@pytest.mark.parametrize("fmt", OQ.SMALL_GROUPS)
@pytest.mark.parametrize("K,N", [(9088, 776), (1024, 264)])
def test_gemv_every_split_and_launch_shape(wq, fmt, K, N):
    W = synth.weight(161, K, N, fmt.startswith("w4"))
    g, _ = quantize_on_gpu(wq, W, fmt)
    P = OQ.pack(fmt, W)
    for M in (1, 3, 7):
        x = synth.activation(161, K, M)
        y_ref = OL.ref_linear(x, P)
        ws = wq.workspace(wq.wq_workspace_size(g, M))
        smax = wq.wq_gemv_max_split(fmt, K)
        for split in [s for s in (1, 2, 4, 8, 32) if s <= smax]:
            assert_parity(_y(wq, g, x, lambda xd, y: wq.wq_gemv(g, xd, y, split, ws=ws)), y_ref,
                          f"{fmt} gemv K={K} M={M} split={split}")
        for rows in (4, 8, 16, 4 | wq.GEMV_PREFETCH, 8 | wq.GEMV_PREFETCH, 16 | wq.GEMV_PREFETCH):
            cap = wq.wq_gemv_max_waves(fmt, M, rows)
            if cap < 1:
                continue
            for waves in sorted({1, cap}):
                assert_parity(_y(wq, g, x, lambda xd, y: wq.wq_gemv_ex(g, xd, y, 2 if K > 4096 else 1, waves, rows,
                                                                       ws=ws)),
                              y_ref, f"{fmt} gemv K={K} M={M} rows={rows:#x} waves={waves}")


@pytest.mark.parametrize("fmt", OQ.SMALL_GROUPS)
def test_gemm_every_tile(wq, fmt):
    K, N = 1024, 520
    W = synth.weight(162, K, N, fmt.startswith("w4"))
    g, _ = quantize_on_gpu(wq, W, fmt)
    P = OQ.pack(fmt, W)
    for M in (8, 13, 40, 300):
        x = synth.activation(162, K, M)
        y_ref = OL.ref_linear(x, P)
        ws = wq.workspace(wq.wq_workspace_size(g, M))
        for tile in range(1, wq.GEMM_TILES + 1):
            assert_parity(_y(wq, g, x, lambda xd, y: wq.wq_gemm(g, xd, y, tile=tile, ws=ws)), y_ref,
                          f"{fmt} gemm M={M} tile={tile}")
        assert_parity(_y(wq, g, x, lambda xd, y: wq.wq_linear(g, xd, y, ws=ws)), y_ref, f"{fmt} linear M={M}")
        # without a workspace the LDS-DMA tiles convert x themselves and split tiles run whole
        assert_parity(_y(wq, g, x, lambda xd, y: wq.wq_gemm(g, xd, y, tile=9, ws=None)), y_ref,
                      f"{fmt} gemm M={M} tile 9 without workspace")


@pytest.mark.parametrize("fmt", OQ.SMALL_GROUPS)
def test_one_hot_is_exact(wq, fmt):
    """A one-hot row of x at either side of a group edge gives bf16 of the exact
    dequantised weight on every path."""
    K, N = 1024, 264
    W = synth.weight(163, K, N, fmt.startswith("w4"))
    g, _ = quantize_on_gpu(wq, W, fmt)
    deq = OQ.dequant(OQ.pack(fmt, W)).T.copy()             # [K][N]
    edges = [0, 31, 32, 63, 64, 95, 127, 128, 511, 512, K - 33, K - 32, K - 1]
    for M, ks in ((3, edges[:3]), (7, edges[3:10]), (13, edges)):
        x = synth.one_hot_activation(K, ks)
        want = OQ.bf16_rne_bits(deq[ks])
        ws = wq.workspace(wq.wq_workspace_size(g, M))
        if M < 8:
            for rows in (4, 8, 16):
                got = _y(wq, g, x, lambda xd, y: wq.wq_gemv_ex(g, xd, y, 1, 0, rows, ws=None))
                assert np.array_equal(got, want), f"{fmt} gemv rows={rows}"
        else:
            for tile in range(1, wq.GEMM_TILES + 1):
                got = _y(wq, g, x, lambda xd, y: wq.wq_gemm(g, xd, y, tile=tile, ws=ws))
                assert np.array_equal(got, want), f"{fmt} gemm tile={tile}"


@pytest.mark.parametrize("fmt", ["w4g32", "w8g64"])
def test_full_decode_shape_and_prefill(wq, fmt):
    """(5120, 27648): every output channel at M = 1 and 4 (tuned GEMV), sampled rows at
    M = 64 and 2048 (the GEMM)."""
    K, N = 5120, 27648
    W = synth.weight(3, K, N, fmt.startswith("w4"))
    g, _ = quantize_on_gpu(wq, W, fmt)
    P = OQ.pack(fmt, W)
    for M in (1, 4):
        x = synth.activation(3, K, M)
        ws = wq.workspace(wq.wq_workspace_size(g, M))
        assert_parity(_y(wq, g, x, lambda xd, y: wq.wq_linear(g, xd, y, ws=ws)), OL.ref_linear(x, P),
                      f"{fmt} M={M}")
    rows = sample_rows(N, 64, seed=3)
    Pr = OQ.pack(fmt, W[rows])
    for M in (64, 2048):
        x = synth.activation(3, K, M)
        ws = wq.workspace(wq.wq_workspace_size(g, M))
        y = _y(wq, g, x, lambda xd, y: wq.wq_linear(g, xd, y, ws=ws))
        assert_parity(y[:, rows], OL.ref_linear(x, Pr), f"{fmt} M={M} sampled rows")


@pytest.mark.parametrize("fmt", OQ.SMALL_GROUPS)
def test_static_and_moe_refusal(wq, fmt):
    """The layer without a workspace (wq_linear_static) bit-identical to wq_linear; the
    grouped (MoE) layer refuses these formats."""
    K, N = 2048, 520
    W = synth.weight(164, K, N, fmt.startswith("w4"))
    g1, _ = quantize_on_gpu(wq, W, fmt)
    for M in (3, 40):
        x = synth.activation(164, K, M)
        ws = wq.workspace(wq.wq_workspace_size(g1, M))
        a = _y(wq, g1, x, lambda xd, y: wq.wq_linear(g1, xd, y, ws=ws))
        b = _y(wq, g1, x, lambda xd, y: wq.wq_linear_static(g1, xd, y))
        assert np.array_equal(a, b), f"{fmt} static M={M}"
        assert_parity(a, OL.ref_linear(x, OQ.pack(fmt, W)), f"{fmt} linear M={M}")
    y = torch.empty((8, N), dtype=torch.bfloat16, device=DEV)
    x = to_dev_bf16(synth.activation(164, K, 8))
    with pytest.raises(wq.WqError) as e:
        wq.wq_moe_linear(g1, x, torch.tensor([0, 8], dtype=torch.int32, device=DEV), y, wq.EPILOGUE_NONE)
    assert e.value.status == 2
