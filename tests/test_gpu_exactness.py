"""GPU: every path multiplies exact dequantised factors, x * q (or x * (q - z)), and
leaves the scale to fp32 sums, so an output carries only the rounding of an fp32 sum
and the final bf16 rounding (reading A12 of the layer: codes stay exact).  Two kinds of
input that an approximate path would fail, each against the oracle:

* large activations whose products cancel: x = +-c over pairs of 128-k blocks holding
  the same codes, so the exact output is 0 while the partial sums are large -- any
  arithmetic that adds a code offset (x (offset + q) - offset sum(x)) or rounds the
  dequantised weight leaves errors far beyond the tolerance here;
* activations below fp16's exact range (|x| ~ 2^-21): a path that rounded them to
  fp16 would change each by up to a few per cent.

Needs an MI355X."""
import numpy as np
import pytest
import torch

import oracle.linear as OL
import oracle.quant as OQ
import synth
from gpu_util import DEV, assert_parity, bf16_bits, quantize_on_gpu, to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wq(wqlib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return wqlib


def _gemv_configs(wq, fmt, M, K):
    """Every (split, waves, rows) launch shape worth covering: the default, every split
    with the default decomposition, and every rows option at 1 and the largest waves."""
    out = [(s, 0, 0) for s in (1, 2, 4) if s <= wq.wq_gemv_max_split(fmt, K)]
    rows_opts = list(wq.ROWS_GRID)
    rows_opts += [r | wq.GEMV_PREFETCH for r in wq.ROWS_GRID if wq.wq_gemv_max_waves(fmt, M, r | wq.GEMV_PREFETCH) > 0]
    rows_opts += [r | wq.GEMV_MFMA for r in (16, 32, 64) if wq.wq_gemv_max_waves(fmt, M, r | wq.GEMV_MFMA) > 0]
    for rows in rows_opts:
        cap = wq.wq_gemv_max_waves(fmt, M, rows)
        for waves in sorted({1, cap}):
            out.append((1, waves, rows))
    return out


def _run_all_gemv(wq, g, x_bits, fmt):
    M, K = x_bits.shape
    xd = to_dev_bf16(x_bits)
    ws = wq.workspace(wq.wq_workspace_size(g, M))
    for split, waves, rows in _gemv_configs(wq, fmt, M, K):
        y = torch.empty((M, g.N), dtype=torch.bfloat16, device=DEV)
        if waves == 0:
            wq.wq_gemv(g, xd, y, split_k=split, ws=ws)
        else:
            wq.wq_gemv_ex(g, xd, y, split, waves, rows, ws=ws)
        torch.cuda.synchronize()
        yield (split, waves, rows), bf16_bits(y)


def _cancelling_case(fmt, K=5120, N=40, M=3, c=256.0):
    """W repeats one random 256-column pattern whose second 128-group equals its first;
    x[m, k] = (-1)^m c for k in the first group of each pair and -(-1)^m c in the
    second, so every pair of groups contributes c s (sum q) - c s (sum q) = 0."""
    rng = np.random.default_rng(7)
    base = (rng.standard_normal((N, 128)) * 0.5).astype(np.float32)
    W = np.tile(np.concatenate([base, base], axis=1), (1, K // 256)).astype(np.float32)
    sign = np.where((np.arange(K) // 128) % 2 == 0, 1.0, -1.0)
    xf = np.stack([((-1.0) ** m) * c * sign for m in range(M)]).astype(np.float32)
    return W, OQ.bf16_rne_bits(xf)


@pytest.mark.parametrize("fmt", OQ.FORMATS + OQ.SMALL_GROUPS)
def test_cancelling_large_activations_gemv(wq, fmt):
    W, x = _cancelling_case(fmt)
    g, _ = quantize_on_gpu(wq, W, fmt)
    P = OQ.pack(fmt, W)
    y_ref = OL.ref_linear(x, P)
    assert np.max(np.abs(y_ref)) == 0.0
    for cfg, y in _run_all_gemv(wq, g, x, fmt):
        assert_parity(y, y_ref, f"{fmt} cancelling gemv {cfg}")
        if fmt == "w8pc":
            # one scale per row: the fp32 sum of c q over the pairs is exactly 0
            assert not np.any(y & 0x7FFF), f"{fmt} {cfg}"


def _tiny_case(fmt, K=5120, N=264, M=4):
    """x ~ 2^-21 N(0, 1) (8 significant bits below fp16's 2^-24 grid) and W scaled so
    that y ~ 1: rounding x to fp16 would cost ~6 % per term."""
    W = (synth.weight(121, K, N, False) * np.float32(2.0 ** 21)).astype(np.float32)
    xf = OQ.bf16_bits_to_f32(synth.activation(121, K, M)) * np.float32(2.0 ** -21)
    return W, OQ.bf16_rne_bits(xf.astype(np.float32))


@pytest.mark.parametrize("fmt", OQ.FORMATS + OQ.SMALL_GROUPS)
def test_tiny_activations_gemv(wq, fmt):
    W, x = _tiny_case(fmt)
    g, _ = quantize_on_gpu(wq, W, fmt)
    P = OQ.pack(fmt, W)
    if fmt == "w4g128":
        assert np.isfinite(P["scales"].astype(np.float32)).all()
    y_ref = OL.ref_linear(x, P)
    assert np.median(np.abs(y_ref)) > 0.3
    for cfg, y in _run_all_gemv(wq, g, x, fmt):
        assert_parity(y, y_ref, f"{fmt} tiny-x gemv {cfg}")


def _gemm_tiles(wq, fmt, K, M):
    return list(range(1, wq.GEMM_TILES + 1))


def _run_gemm_tile(wq, g, x_bits, tile):
    M = x_bits.shape[0]
    y = torch.empty((M, g.N), dtype=torch.bfloat16, device=DEV)
    wq.wq_gemm(g, to_dev_bf16(x_bits), y, tile=tile, ws=wq.workspace(wq.wq_workspace_size(g, M)))
    torch.cuda.synchronize()
    return bf16_bits(y)


@pytest.mark.parametrize("fmt", OQ.FORMATS + OQ.SMALL_GROUPS)
@pytest.mark.parametrize("M", [8, 40, 300])
def test_cancelling_large_activations_gemm(wq, fmt, M):
    W, x = _cancelling_case(fmt, N=264, M=M)
    g, _ = quantize_on_gpu(wq, W, fmt)
    y_ref = OL.ref_linear(x, OQ.pack(fmt, W))
    assert np.max(np.abs(y_ref)) == 0.0
    for tile in _gemm_tiles(wq, fmt, x.shape[1], M):
        y = _run_gemm_tile(wq, g, x, tile)
        assert_parity(y, y_ref, f"{fmt} cancelling gemm M={M} tile={tile}")


@pytest.mark.parametrize("fmt", OQ.FORMATS + OQ.SMALL_GROUPS)
@pytest.mark.parametrize("M", [8, 40, 300])
def test_tiny_activations_gemm(wq, fmt, M):
    W, x = _tiny_case(fmt, M=M)
    g, _ = quantize_on_gpu(wq, W, fmt)
    y_ref = OL.ref_linear(x, OQ.pack(fmt, W))
    for tile in _gemm_tiles(wq, fmt, x.shape[1], M):
        assert_parity(_run_gemm_tile(wq, g, x, tile), y_ref, f"{fmt} tiny-x gemm M={M} tile={tile}")
