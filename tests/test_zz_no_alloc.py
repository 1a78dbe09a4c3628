"""GPU: wq_linear_static, the layer with the library's static scratch (no workspace,
no allocation), against wq_linear with a workspace of wq_workspace_size bytes and
against the oracle: the tuned configurations it meets need partial sums (split-K GEMV,
split-K GEMM), two calls in a row with the second smaller; and a shape whose partial
sums exceed the scratch is refused before any device work.  Needs an MI355X."""
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


def _both(wq, g, x_bits):
    M = x_bits.shape[0]
    x = to_dev_bf16(x_bits)
    y_ref = torch.empty((M, g.N), dtype=torch.bfloat16, device=DEV)
    wq.wq_linear(g, x, y_ref, ws=wq.workspace(wq.wq_workspace_size(g, M)))
    y = torch.full((M, g.N), -7.0, dtype=torch.bfloat16, device=DEV)
    wq.wq_linear_static(g, x, y)
    torch.cuda.synchronize()
    return bf16_bits(y), bf16_bits(y_ref)


@pytest.mark.parametrize("fmt", OQ.FORMATS)
def test_static_scratch_matches_wq_linear(wq, fmt):
    K, N = 4096, 1032
    W = synth.weight(131, K, N, synth.uses_outliers(fmt))
    g, _ = quantize_on_gpu(wq, W, fmt)
    P = OQ.pack(fmt, W)
    try:
        # configurations that write partial sums to the scratch: GEMV split 2-4 at M = 5
        # and 3, GEMM split-K tile 11 at M = 300 and 160
        split = min(4, wq.wq_gemv_max_split(fmt, K))            # 2 for uint4 (2 slices of 2048 k)
        for M in (5, 3):
            wq.wq_tune_cache_set(fmt, K, N, M, wq.KIND_GEMV, wq.gemv_cache_value(split, 2, 8))
        for M in (300, 160):
            wq.wq_tune_cache_set(fmt, K, N, M, wq.KIND_GEMM, 11)
        for pair in ((5, 3), (300, 160)):
            for M in pair:                                   # two calls, the second smaller
                x = synth.activation(131, K, M)
                y, y_lin = _both(wq, g, x)
                assert np.array_equal(y, y_lin), f"{fmt} M={M}"
                assert_parity(y, OL.ref_linear(x, P), f"{fmt} static M={M}")
    finally:
        wq.wq_tune_cache_clear()


def test_static_scratch_refuses_oversized_partials(wq):
    """A GEMV split 32 at M = 7 on a 151936-wide weight needs 32 * 7 * 151936 * 4 bytes
    (136 MB) of partial sums, more than the 64 MiB scratch: refused on the host, nothing
    written.  (The weight is a full-size allocation left uninitialised: it is never read.)"""
    K, N, M = 32768, 151936, 7
    g = wq.PackedWeight("w8pc", wq.GFX950, K, N)
    try:
        wq.wq_tune_cache_set("w8pc", K, N, M, wq.KIND_GEMV, wq.gemv_cache_value(32, 0, 0))
        x = torch.zeros((M, K), dtype=torch.bfloat16, device=DEV)
        y = torch.full((M, N), -7.0, dtype=torch.bfloat16, device=DEV)
        with pytest.raises(wq.WqError, match="static scratch") as e:
            wq.wq_linear_static(g, x, y)
        assert e.value.status == 4 and str(32 * M * N * 4) in str(e.value)
        torch.cuda.synchronize()
        assert torch.all(y == -7.0)
    finally:
        wq.wq_tune_cache_clear()
