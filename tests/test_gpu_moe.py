"""GPU: the grouped (mixture-of-experts) layer and its SiLU-gated epilogue through the
C ABI against the oracle (oracle/moe.py): every format, an expert without rows, an
expert with more than one block of 16 rows, activations that fp16 cannot hold exactly,
offsets beyond the row count (clamped), the dense case (one expert), and graph replay.
Needs an MI355X."""
import numpy as np
import pytest
import torch

import oracle.moe as OM
import oracle.quant as OQ
import synth
from gpu_util import DEV, assert_parity, bf16_bits, to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wq(wqlib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return wqlib


def _experts(wq, fmt, E, K, N, seed):
    Ws = [synth.weight(seed + e, K, N, synth.uses_outliers(fmt)) for e in range(E)]
    g = wq.quantize_experts([torch.from_numpy(W).to(DEV) for W in Ws], fmt)
    torch.cuda.synchronize()
    return g, [OQ.pack(fmt, W) for W in Ws]


def _run(wq, g, x_bits, off, gated):
    T = x_bits.shape[0]
    width = g.N // 2 if gated else g.N
    y = torch.full((T, width), -3.0, dtype=torch.bfloat16, device=DEV)
    wq.wq_moe_linear(g, to_dev_bf16(x_bits), torch.from_numpy(np.asarray(off, np.int32)).to(DEV), y,
                     wq.EPILOGUE_SILU_MUL if gated else wq.EPILOGUE_NONE)
    torch.cuda.synchronize()
    return bf16_bits(y)


@pytest.mark.parametrize("fmt", OQ.FORMATS)
@pytest.mark.parametrize("gated", [False, True])
def test_moe_against_oracle(wq, fmt, gated):
    E, K, N, T = 6, 1024, 96, 41
    off = [0, 3, 3, 24, 30, 31, 41]          # expert 1 empty, expert 2 spans two 16-row blocks
    g, Ps = _experts(wq, fmt, E, K, N, seed=140)
    x = synth.activation(140, K, T)
    ref = OM.ref_moe_silu_mul(x, off, Ps) if gated else OM.ref_moe_linear(x, off, Ps)
    assert_parity(_run(wq, g, x, off, gated), ref, f"moe {fmt} gated={gated}")


@pytest.mark.parametrize("fmt", OQ.FORMATS)
@pytest.mark.parametrize("T,off", [
    (90, [0, 25, 25, 58, 90]),            # 22.5 rows per expert: two blocks per pass; 25 = a partial second block
    (260, [0, 1, 113, 200, 260]),         # 65 per expert: four blocks per pass; 112 = 1 3/4 groups of 64, 87 with a lone last row
    (420, [0, 130, 130, 300, 420]),       # 105 per expert: eight blocks per pass; 130 = a group of 128 and 2 rows
])
def test_moe_token_blocks_per_pass(wq, fmt, T, off):
    """More rows per expert: each unit's codes feed two, four or eight 16-row blocks per pass
    over the weights (chosen from the average rows per expert), with partly filled
    blocks and groups, an empty expert and one with a single row; both epilogues; an
    fp16-inexact x in one block."""
    E, K, N = 4, 640, 64
    g, Ps = _experts(wq, fmt, E, K, N, seed=144)
    xf = OQ.bf16_bits_to_f32(synth.activation(144, K, T)).copy()
    xf[T - 2, 300] = 1.0e-7                                      # one unit of one block on the exact path
    x = OQ.bf16_rne_bits(xf.astype(np.float32))
    for gated in (False, True):
        ref = OM.ref_moe_silu_mul(x, off, Ps) if gated else OM.ref_moe_linear(x, off, Ps)
        assert_parity(_run(wq, g, x, off, gated), ref, f"moe {fmt} T={T} gated={gated}")


@pytest.mark.parametrize("fmt", OQ.FORMATS)
def test_moe_activations_fp16_cannot_hold(wq, fmt):
    """Units with |x| > 65280 or 0 < |x| < 2^-17 take the exact bf16 path."""
    E, K, N, T = 3, 1024, 64, 20
    off = [0, 7, 12, 20]
    g, Ps = _experts(wq, fmt, E, K, N, seed=141)
    xf = OQ.bf16_bits_to_f32(synth.activation(141, K, T)).copy()
    xf[2, 100] = 3.0e5
    xf[9, 700] = 3.0e-7
    xf[15, 5] = -65280.0
    x = OQ.bf16_rne_bits(xf.astype(np.float32))
    for gated in (False, True):
        ref = OM.ref_moe_silu_mul(x, off, Ps) if gated else OM.ref_moe_linear(x, off, Ps)
        assert_parity(_run(wq, g, x, off, gated), ref, f"moe {fmt} gated={gated} big/tiny x")


def test_moe_dense_and_clamped_offsets(wq):
    """One expert over all rows is the dense layer (wq_linear's result within the
    tolerance of the same oracle); offsets past T are clamped to T; rows outside every
    range are left untouched."""
    fmt, K, N, T = "w4g128", 2048, 128, 9
    g, Ps = _experts(wq, fmt, 1, K, N, seed=142)
    x = synth.activation(142, K, T)
    assert_parity(_run(wq, g, x, [0, T], False), OM.ref_moe_linear(x, [0, T], Ps), "dense")
    g2, Ps2 = _experts(wq, fmt, 2, K, N, seed=143)
    y = _run(wq, g2, x, [2, 5, T + 100], False)             # rows 0, 1 in no range
    assert np.all(y[:2] == OQ.bf16_rne_bits(np.float32(-3.0)))
    ref = OM.ref_moe_linear(x[2:], [0, 3, T - 2], Ps2)
    assert_parity(y[2:], ref, "clamped offsets")


def test_moe_graph_replay(wq):
    fmt, E, K, N, T = "w8g128", 4, 1024, 64, 12
    g, Ps = _experts(wq, fmt, E, K, N, seed=144)
    x = synth.activation(144, K, T)
    off = [0, 2, 6, 6, 12]
    xd = to_dev_bf16(x)
    od = torch.tensor(off, dtype=torch.int32, device=DEV)
    y = torch.empty((T, N // 2), dtype=torch.bfloat16, device=DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        wq.wq_moe_linear(g, xd, od, y, wq.EPILOGUE_SILU_MUL, stream=s)
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr, stream=s):
            wq.wq_moe_linear(g, xd, od, y, wq.EPILOGUE_SILU_MUL, stream=s)
    ref = OM.ref_moe_silu_mul(x, off, Ps)
    first = None
    for _ in range(3):
        y.fill_(0)
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        yb = bf16_bits(y)
        assert_parity(yb, ref, "graph replay")
        first = yb if first is None else first
        assert np.array_equal(yb, first)
