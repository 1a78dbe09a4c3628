"""GPU: INT4 per output channel (WQ_FMT_W4_PC) through the C ABI against the oracle
(oracle/quant.py, "w4pc"): bit-exact packing from fp32 and bf16 weights, the gfx950
layout that repeats each row's scale and zero-point in every 128-k group and its exact
inverse, the GEMV at every split and launch shape, every GEMM tile, one-hot inputs, the
full (5120, 27648) decode shape, the tuned layer, the grouped (MoE) layer and the
no-allocation entry point.  Needs an MI355X."""
import numpy as np
import pytest
import torch

import oracle.linear as OL
import oracle.moe as OM
import oracle.quant as OQ
import synth
from gpu_util import (DEV, assert_parity, bf16_bits, canonical_to_host, quantize_on_gpu, sample_rows,
                      to_dev_bf16)

pytestmark = pytest.mark.gpu
FMT = "w4pc"


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


@pytest.mark.parametrize("K,N", [(1024, 264), (640, 40), (128, 8)])
def test_pack_repack_bitexact(wq, K, N):
    W = synth.weight(150, K, N, True)
    W[3] = 0                                      # an all-zero row
    W[5] = np.float32(0.5)                        # a constant row: s = 0, dequant 0
    g, can = quantize_on_gpu(wq, W, FMT)
    got, want = canonical_to_host(can, FMT), OQ.pack(FMT, W)
    for key in ("qweight", "scales", "zeros"):
        assert np.array_equal(got[key].view(np.uint8), want[key].view(np.uint8)), key
    # bf16 weights pack as the oracle packs their exact fp32 widening
    Wb = OQ.bf16_rne_bits(W)
    Wt = torch.from_numpy(Wb.view(np.int16)).to(DEV).view(torch.bfloat16)
    gb, canb = wq.quantize(Wt, FMT, keep_canonical=True)
    gotb, wantb = canonical_to_host(canb, FMT), OQ.pack(FMT, OQ.bf16_bits_to_f32(Wb))
    for key in ("qweight", "scales", "zeros"):
        assert np.array_equal(gotb[key].view(np.uint8), wantb[key].view(np.uint8)), "bf16 " + key
    # the gfx950 metadata repeats each row's scale and zero-point in every group
    G = K // 128
    st = g.scales.cpu().numpy().view(np.uint16).reshape(-1, G, 16)
    assert np.all(st == st[:, :1, :])
    zt = g.zeros.cpu().numpy().reshape(-1, G, 8)
    assert np.all(zt == zt[:, :1, :])
    back = wq.PackedWeight(FMT, wq.CANONICAL, K, N)
    wq.wq_unrepack(g, back)
    torch.cuda.synchronize()
    for a, b in ((back.qweight, can.qweight), (back.scales, can.scales), (back.zeros, can.zeros)):
        assert torch.equal(a, b)


@pytest.mark.parametrize("K,N", [(9088, 776), (1024, 264)])
def test_gemv_every_split_and_launch_shape(wq, K, N):
    W = synth.weight(151, K, N, True)
    g, _ = quantize_on_gpu(wq, W, FMT)
    P = OQ.pack(FMT, W)
    for M in (1, 3, 7):
        x = synth.activation(151, K, M)
        y_ref = OL.ref_linear(x, P)
        ws = wq.workspace(wq.wq_workspace_size(g, M))
        smax = wq.wq_gemv_max_split(FMT, K)
        for split in [s for s in (1, 2, 4, 8, 32) if s <= smax]:
            assert_parity(_y(wq, g, x, lambda xd, y: wq.wq_gemv(g, xd, y, split, ws=ws)), y_ref,
                          f"gemv K={K} M={M} split={split}")
        for rows in (4, 8, 16, 16 | wq.GEMV_MFMA, 32 | wq.GEMV_MFMA, 64 | wq.GEMV_MFMA):
            if wq.wq_gemv_max_waves(FMT, M, rows) < 1:
                continue
            assert_parity(_y(wq, g, x, lambda xd, y: wq.wq_gemv_ex(g, xd, y, 1, 0, rows, ws=None)), y_ref,
                          f"gemv K={K} M={M} rows={rows:#x}")


def test_gemm_every_tile(wq):
    K, N = 1024, 520
    W = synth.weight(152, K, N, True)
    g, _ = quantize_on_gpu(wq, W, FMT)
    P = OQ.pack(FMT, W)
    for M in (8, 13, 40, 300):
        x = synth.activation(152, K, M)
        y_ref = OL.ref_linear(x, P)
        ws = wq.workspace(wq.wq_workspace_size(g, M))
        for tile in range(1, wq.GEMM_TILES + 1):
            assert_parity(_y(wq, g, x, lambda xd, y: wq.wq_gemm(g, xd, y, tile=tile, ws=ws)), y_ref,
                          f"gemm M={M} tile={tile}")
        assert_parity(_y(wq, g, x, lambda xd, y: wq.wq_linear(g, xd, y, ws=ws)), y_ref, f"linear M={M}")


def test_one_hot_is_exact(wq):
    """A one-hot row of x gives bf16 of the exact dequantised weight on every path."""
    K, N = 1024, 264
    W = synth.weight(153, K, N, True)
    g, _ = quantize_on_gpu(wq, W, FMT)
    deq = OQ.dequant(OQ.pack(FMT, W)).T.copy()             # [K][N]
    for M, ks in ((3, [0, 511, K - 1]), (9, list(range(0, K, 120))[:9])):
        x = synth.one_hot_activation(K, ks)
        want = OQ.bf16_rne_bits(deq[ks])
        ws = wq.workspace(wq.wq_workspace_size(g, M))
        if M < 8:
            for rows in (4, 16 | wq.GEMV_MFMA):
                got = _y(wq, g, x, lambda xd, y: wq.wq_gemv_ex(g, xd, y, 1, 0, rows, ws=None))
                assert np.array_equal(got, want), f"gemv rows={rows:#x}"
        else:
            for tile in range(1, wq.GEMM_TILES + 1):
                got = _y(wq, g, x, lambda xd, y: wq.wq_gemm(g, xd, y, tile=tile, ws=ws))
                assert np.array_equal(got, want), f"gemm tile={tile}"


def test_full_decode_shape_and_prefill(wq):
    """(5120, 27648): every output channel at M = 1 and 4 (tuned GEMV), sampled rows at
    M = 64 and 2048 (the GEMM)."""
    K, N = 5120, 27648
    W = synth.weight(3, K, N, True)
    g, _ = quantize_on_gpu(wq, W, FMT)
    P = OQ.pack(FMT, W)
    for M in (1, 4):
        x = synth.activation(3, K, M)
        ws = wq.workspace(wq.wq_workspace_size(g, M))
        assert_parity(_y(wq, g, x, lambda xd, y: wq.wq_linear(g, xd, y, ws=ws)), OL.ref_linear(x, P),
                      f"M={M}")
    rows = sample_rows(N, 64, seed=3)
    Pr = OQ.pack(FMT, W[rows])
    for M in (64, 2048):
        x = synth.activation(3, K, M)
        ws = wq.workspace(wq.wq_workspace_size(g, M))
        y = _y(wq, g, x, lambda xd, y: wq.wq_linear(g, xd, y, ws=ws))
        assert_parity(y[:, rows], OL.ref_linear(x, Pr), f"M={M} sampled rows")


def test_moe_and_static(wq):
    """Per-channel W4 experts in the grouped layer (both epilogues), and the layer
    without a workspace (wq_linear_static) bit-identical to wq_linear."""
    E, K, N, T = 3, 1024, 64, 30
    Ws = [synth.weight(154 + e, K, N, True) for e in range(E)]
    g = wq.quantize_experts([torch.from_numpy(W).to(DEV) for W in Ws], FMT)
    Ps = [OQ.pack(FMT, W) for W in Ws]
    off = [0, 11, 11, 30]
    x = synth.activation(154, K, T)
    for gated in (False, True):
        width = N // 2 if gated else N
        y = torch.empty((T, width), dtype=torch.bfloat16, device=DEV)
        wq.wq_moe_linear(g, to_dev_bf16(x), torch.tensor(off, dtype=torch.int32, device=DEV), y,
                         wq.EPILOGUE_SILU_MUL if gated else wq.EPILOGUE_NONE)
        torch.cuda.synchronize()
        ref = OM.ref_moe_silu_mul(x, off, Ps) if gated else OM.ref_moe_linear(x, off, Ps)
        assert_parity(bf16_bits(y), ref, f"moe gated={gated}")
    K, N = 2048, 520
    W = synth.weight(155, K, N, True)
    g1, _ = quantize_on_gpu(wq, W, FMT)
    for M in (3, 40):
        x = synth.activation(155, K, M)
        ws = wq.workspace(wq.wq_workspace_size(g1, M))
        a = _y(wq, g1, x, lambda xd, y: wq.wq_linear(g1, xd, y, ws=ws))
        b = _y(wq, g1, x, lambda xd, y: wq.wq_linear_static(g1, xd, y))
        assert np.array_equal(a, b), f"static M={M}"
        assert_parity(a, OL.ref_linear(x, OQ.pack(FMT, W)), f"linear M={M}")
