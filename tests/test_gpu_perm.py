"""The layer with the full-K activation permutation through the C ABI against the
oracle: the weight is stored with its columns in the order perm (W[:, perm],
quantised and packed on the GPU), the activations are gathered by the same perm
inside the call, and the result matches the oracle's x[:, perm] . dequant(W')^T
within the layer's tolerance -- and bit for bit the plain layer on activations
gathered by torch, since the same kernels run on the same x'."""
import numpy as np
import pytest
import torch

import oracle.linear as OL
import oracle.quant as OQ
import synth
from gpu_util import (DEV, assert_parity, bf16_bits, host_weight, oracle_pack_rows, quantize_on_gpu,
                      sample_rows, to_dev_bf16)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wq(wqlib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return wqlib


def _perm(seed, K, bad=False):
    p = np.random.default_rng(seed).permutation(K).astype(np.int32)
    if bad:                                   # out-of-range entries read +0; repeats gather twice
        p[3], p[K - 1], p[7] = K, -5, p[8]
    return p


def _run_perm(wq, g, x_bits, perm):
    M = x_bits.shape[0]
    y = torch.empty((M, g.N), dtype=torch.bfloat16, device=DEV)
    ws = wq.workspace(wq.wq_linear_perm_workspace_size(g, M))
    wq.wq_linear_perm(g, to_dev_bf16(x_bits), torch.from_numpy(perm).to(DEV), y, ws)
    torch.cuda.synchronize()
    return bf16_bits(y)


def _run_plain(wq, g, x_bits):
    M = x_bits.shape[0]
    y = torch.empty((M, g.N), dtype=torch.bfloat16, device=DEV)
    wq.wq_linear(g, to_dev_bf16(x_bits), y, ws=wq.workspace(wq.wq_workspace_size(g, M)))
    torch.cuda.synchronize()
    return bf16_bits(y)


@pytest.mark.parametrize("fmt,K,N", [("w8pc", 384, 264), ("w8g128", 384, 264), ("w4g128", 1024, 520),
                                     ("w8pc", 2320, 200)])
@pytest.mark.parametrize("bad", [False, True])
def test_linear_perm_against_oracle(wq, fmt, K, N, bad):
    """GEMV and GEMM token counts, a ragged K slice (K = 2320), a true permutation and
    one with out-of-range and repeated indices."""
    W = synth.weight(301, K, N, synth.uses_outliers(fmt))
    perm = _perm(301 + K, K, bad)
    Wp = np.ascontiguousarray(W[:, np.clip(perm, 0, K - 1)])
    g, _ = quantize_on_gpu(wq, Wp, fmt)
    P = OQ.pack(fmt, Wp)
    for M in (1, 4, 7, 8, 37, 300):
        x = synth.activation(301, K, M)
        y = _run_perm(wq, g, x, perm)
        assert_parity(y, OL.ref_linear_perm(x, P, perm), f"perm {fmt} K={K} N={N} M={M} bad={bad}")
        # the same kernels on the gathered activations, bit for bit
        assert np.array_equal(y, _run_plain(wq, g, OL.gather_activations(x, perm))), (fmt, M)
    # an index array that is 4- but not 16-byte aligned takes the scalar index loads
    x = synth.activation(302, K, 3)
    buf = torch.zeros(K + 1, dtype=torch.int32, device=DEV)
    buf[1:] = torch.from_numpy(perm).to(DEV)
    pv = buf[1:]
    assert pv.data_ptr() % 16 != 0
    y = torch.empty((3, N), dtype=torch.bfloat16, device=DEV)
    wq.wq_linear_perm(g, to_dev_bf16(x), pv, y, wq.workspace(wq.wq_linear_perm_workspace_size(g, 3)))
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(y), _run_perm(wq, g, x, perm))


def test_linear_perm_restores_the_plain_layer(wq):
    """Per-channel codes do not depend on the column order, so storing W[:, perm] and
    gathering x by perm gives the plain layer's products in another summation order:
    equal to it within the tolerance, for the GEMV and the GEMM."""
    K, N = 2048, 520
    W = synth.weight(302, K, N)
    perm = _perm(302, K)
    g0, _ = quantize_on_gpu(wq, W, "w8pc")
    g1, _ = quantize_on_gpu(wq, np.ascontiguousarray(W[:, perm]), "w8pc")
    P = OQ.pack("w8pc", W)
    for M in (1, 5, 64):
        x = synth.activation(302, K, M)
        y_ref = OL.ref_linear(x, P)
        assert_parity(_run_perm(wq, g1, x, perm), y_ref, f"perm restores M={M}")
        assert_parity(_run_plain(wq, g0, x), y_ref, f"plain M={M}")


@pytest.mark.parametrize("cfg,fmt,K,N", [(3, "w4g128", 5120, 27648), (5, "w8pc", 5120, 27648)])
def test_linear_perm_full_size(wq, cfg, fmt, K, N):
    """The decode and prefill shapes: sampled rows against the oracle, and every output
    bit for bit against the plain layer on gathered activations."""
    W = host_weight(cfg, K, N, synth.uses_outliers(fmt))
    perm = _perm(cfg, K)
    Wp = np.ascontiguousarray(W[:, perm])
    g, _ = quantize_on_gpu(wq, Wp, fmt)
    rows = sample_rows(N, 64, seed=cfg)
    P = oracle_pack_rows(fmt, Wp, rows)
    for M in ((1, 4) if fmt == "w4g128" else (8, 2048)):
        x = synth.activation(cfg, K, M)
        y = _run_perm(wq, g, x, perm)
        assert_parity(y[:, rows], OL.ref_linear_perm(x, P, perm), f"perm full {fmt} M={M}")
        assert np.array_equal(y, _run_plain(wq, g, OL.gather_activations(x, perm))), (fmt, M)
