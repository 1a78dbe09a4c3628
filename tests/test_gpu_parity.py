"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the same
seeded inputs.  Packed bytes must be bit-exact; every bf16 output element must
satisfy |y - y_ref| <= 1e-2 * max(1, |y_ref|); one-hot and identity inputs must
reproduce the dequantised weights bit-exactly.  Needs an MI355X."""
import numpy as np
import pytest
import torch

import oracle.linear as OL
import oracle.quant as OQ
import synth
from gpu_util import (DEV, assert_parity, bf16_bits, canonical_to_host, host_weight, oracle_pack_rows,
                      quantize_on_gpu, sample_rows, to_dev_bf16)

pytestmark = pytest.mark.gpu

SPLITS = (1, 2, 4, 8, 16, 32)


@pytest.fixture(scope="module")
def wq(wqlib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return wqlib


def _allowed_splits(fmt, K):
    import gemm_decode_amd.wq as wqb
    return [s for s in SPLITS if s <= wqb.wq_gemv_max_split(fmt, K)]


def _run_gemv(wq, g, x_bits, split):
    M = x_bits.shape[0]
    x = to_dev_bf16(x_bits)
    y = torch.empty((M, g.N), dtype=torch.bfloat16, device=DEV)
    ws = wq.workspace(wq.wq_workspace_size(g, M))
    wq.wq_gemv(g, x, y, split_k=split, ws=ws)
    torch.cuda.synchronize()
    return bf16_bits(y)


def _rows_options(wq, fmt, M):
    """Rows per wave, each also with the slice-prefetch flag where it is offered, and
    the matrix-core GEMV's tiles per workgroup where it is offered."""
    out = []
    for rows in wq.ROWS_GRID:
        out.append(rows)
        if wq.wq_gemv_max_waves(fmt, M, rows | wq.GEMV_PREFETCH) > 0:
            out.append(rows | wq.GEMV_PREFETCH)
    for rows in (16, 32, 64):
        if wq.wq_gemv_max_waves(fmt, M, rows | wq.GEMV_MFMA) > 0:
            out.append(rows | wq.GEMV_MFMA)
    return out


def _selected(fmt, tile, w):
    """bf16 bits a path returns when x selects the dequantised weights w exactly: every
    path multiplies exact codes and scales fp32 sums, so bf16(w) on every tile."""
    return OQ.bf16_rne_bits(np.ascontiguousarray(w, dtype=np.float32))


def _run_gemm(wq, g, x_bits, tile=0, with_ws=True):
    M = x_bits.shape[0]
    x = to_dev_bf16(x_bits)
    y = torch.empty((M, g.N), dtype=torch.bfloat16, device=DEV)
    # split-K partials; for group-128 LDS-DMA tiles also x in fp16
    ws = wq.workspace(wq.wq_workspace_size(g, M)) if with_ws else None
    wq.wq_gemm(g, x, y, tile=tile, ws=ws)
    torch.cuda.synchronize()
    return bf16_bits(y)


# ------------------------------------------------------------------ packing
@pytest.mark.parametrize("fmt", OQ.FORMATS)
def test_pack_bf16_input_bitexact(wq, fmt):
    """wq_pack_bf16: a bf16 weight packs exactly as the oracle packs its (exact) fp32
    widening; ragged K groups and N rows across several blocks."""
    K, N = 1280, 776
    W = synth.weight(109, K, N, synth.uses_outliers(fmt))
    Wb = OQ.bf16_rne_bits(W)                                   # the checkpoint's bf16 bits
    Wf = OQ.bf16_bits_to_f32(Wb)                               # their exact widening
    P = OQ.pack(fmt, Wf)
    wt = torch.from_numpy(Wb.view(np.int16)).to(DEV).view(torch.bfloat16)
    g, can = wq.quantize(wt, fmt, keep_canonical=True)
    got = canonical_to_host(can, fmt)
    for key in ("qweight", "scales") + (("zeros",) if fmt == "w4g128" else ()):
        assert np.array_equal(got[key].view(np.uint8), np.ascontiguousarray(P[key]).view(np.uint8)), key
    x = synth.activation(109, K, 3)
    assert_parity(_run_gemv(wq, g, x, 1), OL.ref_linear(x, P), f"{fmt} bf16-packed gemv")


SMALL = [("w8pc", 1024, 1024), ("w8pc", 2320, 1000), ("w8g128", 1280, 1000), ("w4g128", 1280, 776),
         ("w8g128", 384, 264), ("w4g128", 384, 264), ("w8pc", 5200, 1000), ("w4g128", 9088, 264)]


@pytest.mark.parametrize("fmt,K,N", SMALL)
def test_pack_bitexact_small(wq, fmt, K, N):
    W = synth.weight(91, K, N, synth.uses_outliers(fmt))
    W[3] = 0                                      # an all-zero row
    W[5, :128] = 0                                # an all-zero group
    g, can = quantize_on_gpu(wq, W, fmt)
    got, want = canonical_to_host(can, fmt), OQ.pack(fmt, W)
    for key in ("qweight", "scales", "zeros"):
        if key in want:
            assert np.array_equal(got[key].view(np.uint8), want[key].view(np.uint8)), key
    back = wq.PackedWeight(fmt, wq.CANONICAL, K, N)
    wq.wq_unrepack(g, back)
    torch.cuda.synchronize()
    for a, b in ((back.qweight, can.qweight), (back.scales, can.scales), (back.zeros, can.zeros)):
        if a is not None:
            assert torch.equal(a, b)


BIG = [(2, "w8pc", 5120, 27648), (2, "w8pc", 13824, 5120), (2, "w8pc", 5120, 7168),
       (2, "w8pc", 6144, 5120), (3, "w4g128", 5120, 27648), (3, "w4g128", 13824, 5120),
       (4, "w8pc", 27648, 5120), (4, "w8g128", 27648, 5120), (4, "w4g128", 27648, 5120),
       (4, "w8pc", 5120, 151936), (4, "w8g128", 5120, 151936), (4, "w4g128", 5120, 151936)]


def _big_case(wq, cfg, fmt, K, N):
    W = host_weight(cfg, K, N, synth.uses_outliers(fmt))
    g, can = quantize_on_gpu(wq, W, fmt)
    rows = sample_rows(N, 64, seed=cfg)
    return W, g, can, rows


@pytest.mark.parametrize("cfg,fmt,K,N", BIG)
def test_full_size_pack_and_gemv(wq, cfg, fmt, K, N):
    """Full-size weights in the configuration the bench times: canonical bytes
    bit-exact on every row; GEMV (tuned default and every split) on every output
    channel against the oracle, which packs the same fp32 weight itself."""
    W = host_weight(cfg, K, N, synth.uses_outliers(fmt))
    g, can = quantize_on_gpu(wq, W, fmt)
    got = canonical_to_host(can, fmt)
    want = OQ.pack(fmt, W)
    for key in ("qweight", "scales") + (("zeros",) if fmt == "w4g128" else ()):
        assert np.array_equal(got[key].view(np.uint8), np.ascontiguousarray(want[key]).view(np.uint8)), key
    del got, can
    Ms = synth.CONFIGS[cfg]["Ms"]
    splits = [0] + (_allowed_splits(fmt, K) if cfg == 4 else [1])
    for M in Ms:
        x = synth.activation(cfg, K, M)
        y_ref = OL.ref_linear(x, want)
        for split in splits:
            y = _run_gemv(wq, g, x, split)
            assert_parity(y, y_ref, f"{fmt} K={K} N={N} M={M} split={split}")


GEMM_BIG = [(5, "w8pc", 5120, 27648), (5, "w8pc", 13824, 5120), (5, "w4g128", 5120, 27648),
            (5, "w4g128", 13824, 5120)]


@pytest.mark.parametrize("cfg,fmt,K,N", GEMM_BIG)
def test_full_size_gemm(wq, cfg, fmt, K, N):
    W, g, can, rows = _big_case(wq, cfg, fmt, K, N)
    want = oracle_pack_rows(fmt, W, rows)
    for M in (8, 16, 64, 128, 512, 2048):
        x = synth.activation(cfg, K, M)
        y_ref = OL.ref_linear(x, want)
        for tile in range(1, wq.GEMM_TILES + 1):
            y = _run_gemm(wq, g, x, tile)
            assert_parity(y[:, rows], y_ref, f"gemm {fmt} K={K} N={N} M={M} tile={tile}")
        yl = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
        wq.wq_linear(g, to_dev_bf16(x), yl)
        torch.cuda.synchronize()
        assert_parity(bf16_bits(yl)[:, rows], y_ref, f"linear {fmt} M={M}")


# ------------------------------------------------------------- small, full
@pytest.mark.parametrize("fmt,K,N", [("w8pc", 5200, 1000), ("w8g128", 9088, 1000), ("w4g128", 9088, 776)])
def test_gemv_every_split_and_waves(wq, fmt, K, N):
    """Both levels of the K split: every (split_k, waves per workgroup) pair."""
    W = synth.weight(90, K, N, synth.uses_outliers(fmt))
    g, can = quantize_on_gpu(wq, W, fmt)
    P = OQ.pack(fmt, W)
    for M in (1, 3, 7):
        xb = synth.activation(90, K, M)
        y_ref = OL.ref_linear(xb, P)
        x = to_dev_bf16(xb)
        ws = wq.workspace(wq.wq_workspace_size(g, M))
        for split in _allowed_splits(fmt, K):
            for rows in _rows_options(wq, fmt, M):
                cap = wq.wq_gemv_max_waves(fmt, M, rows)
                for waves in sorted(set(v for v in (1, 2, 3, 5, cap) if v <= cap)):
                    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
                    wq.wq_gemv_ex(g, x, y, split, waves, rows, ws=ws)
                    torch.cuda.synchronize()
                    assert_parity(bf16_bits(y), y_ref, f"gemv {fmt} M={M} split={split} rows={rows} waves={waves}")


@pytest.mark.parametrize("fmt,K,N", SMALL)
def test_gemv_small_every_m_and_split(wq, fmt, K, N):
    W = synth.weight(92, K, N, synth.uses_outliers(fmt))
    g, can = quantize_on_gpu(wq, W, fmt)
    P = OQ.pack(fmt, W)
    for M in range(1, 8):
        x = synth.activation(92, K, M)
        y_ref = OL.ref_linear(x, P)
        for split in [0] + _allowed_splits(fmt, K):
            assert_parity(_run_gemv(wq, g, x, split), y_ref, f"gemv {fmt} M={M} split={split}")


@pytest.mark.parametrize("fmt,K,N", [("w8pc", 384, 264), ("w8g128", 384, 264), ("w4g128", 384, 264),
                                     ("w8pc", 1040, 200), ("w4g128", 1024, 520)])
@pytest.mark.parametrize("M", [1, 7, 8, 37, 150, 300])
def test_gemm_small(wq, fmt, K, N, M):
    W = synth.weight(93, K, N, synth.uses_outliers(fmt))
    g, can = quantize_on_gpu(wq, W, fmt)
    x = synth.activation(93, K, M)
    y_ref = OL.ref_linear(x, OQ.pack(fmt, W))
    for tile in range(1, wq.GEMM_TILES + 1):
        assert_parity(_run_gemm(wq, g, x, tile), y_ref, f"gemm {fmt} K={K} N={N} M={M} tile={tile}")
    if fmt != "w8pc":   # tile 9 without the workspace's fp16 x: converts in LDS, same bits
        assert np.array_equal(_run_gemm(wq, g, x, 9, with_ws=False), _run_gemm(wq, g, x, 9))


EDGE = [("w8pc", 16, 8), ("w4g128", 128, 8), ("w8g128", 128, 24), ("w8pc", 64, 17),
        ("w8pc", 2176, 300), ("w8pc", 4160, 272), ("w4g128", 2176, 136)]


@pytest.mark.parametrize("fmt,K,N", EDGE)
def test_edge_shapes_every_path(wq, fmt, K, N):
    """Boundary shapes on every path: minimum K and N, a short last 16-row tile, a lone
    row in it, a ragged 1 KB slice, DMA K steps that leave 1 or 2 steps after the
    three-step loop, and M at the edges of the 16-, 32-, 128- and 256-row tiles (13: a
    16-token A operand that is partly filled)."""
    W = synth.weight(96, K, N, synth.uses_outliers(fmt))
    g, can = quantize_on_gpu(wq, W, fmt)
    P = OQ.pack(fmt, W)
    for M in (1, 5, 7, 8, 13, 16, 17, 33, 64, 128, 129, 257):
        x = synth.activation(96, K, M)
        y_ref = OL.ref_linear(x, P)
        if M < 8:
            for split in [0] + _allowed_splits(fmt, K):
                assert_parity(_run_gemv(wq, g, x, split), y_ref, f"gemv {fmt} K={K} N={N} M={M} split={split}")
            xd = to_dev_bf16(x)
            for rows in (16 | wq.GEMV_MFMA, 64 | wq.GEMV_MFMA):   # ragged 128-k units, short tiles
                for waves in (1, 3):
                    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
                    wq.wq_gemv_ex(g, xd, y, 1, waves, rows, ws=None)
                    torch.cuda.synchronize()
                    assert_parity(bf16_bits(y), y_ref, f"gemv {fmt} K={K} N={N} M={M} rows={rows} waves={waves}")
        for tile in range(1, wq.GEMM_TILES + 1):
            assert_parity(_run_gemm(wq, g, x, tile), y_ref, f"gemm {fmt} K={K} N={N} M={M} tile={tile}")
        yl = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
        ws = wq.workspace(wq.wq_workspace_size(g, M))
        wq.wq_linear(g, to_dev_bf16(x), yl, ws=ws)
        torch.cuda.synchronize()
        assert_parity(bf16_bits(yl), y_ref, f"linear {fmt} K={K} N={N} M={M}")


# ---------------------------------------------------------- exact special inputs
@pytest.mark.parametrize("fmt", OQ.FORMATS)
def test_one_hot_is_exact(wq, fmt):
    """x = e_k: every path returns bf16(dequant(W)[n, k]) bit-exactly (one exact
    nonzero term in every fp32 sum), for every split, every waves count and every
    GEMM tile.  K spans several (and a ragged) K slices."""
    K, N = 9216, 264
    W = synth.weight(94, K, N, synth.uses_outliers(fmt))
    g, can = quantize_on_gpu(wq, W, fmt)
    P = OQ.pack(fmt, W)
    ks = [0, 127, 128, 4999, 5120, K - 1]
    x = synth.one_hot_activation(K, ks)
    want = OQ.bf16_rne_bits(OQ.dequant(P)[:, ks].T.astype(np.float32))
    for split in _allowed_splits(fmt, K):
        assert np.array_equal(_run_gemv(wq, g, x, split), want), f"gemv split={split}"
    xd = to_dev_bf16(x)
    ws = wq.workspace(wq.wq_workspace_size(g, len(ks)))
    for rows in _rows_options(wq, fmt, len(ks)):
        for waves in range(1, wq.wq_gemv_max_waves(fmt, len(ks), rows) + 1):
            for split in (1, 2):
                y = torch.empty((len(ks), N), dtype=torch.bfloat16, device=DEV)
                wq.wq_gemv_ex(g, xd, y, split, waves, rows, ws=ws)
                torch.cuda.synchronize()
                assert np.array_equal(bf16_bits(y), want), f"gemv split={split} rows={rows} waves={waves}"
    for tile in range(1, wq.GEMM_TILES + 1):
        assert np.array_equal(_run_gemm(wq, g, x, tile), _selected(fmt, tile, OQ.dequant(P)[:, ks].T)), \
            f"gemm tile={tile}"


@pytest.mark.parametrize("fmt", OQ.FORMATS)
def test_identity_is_exact(wq, fmt):
    K, N = 1024, 264
    W = synth.weight(95, K, N, synth.uses_outliers(fmt))
    g, can = quantize_on_gpu(wq, W, fmt)
    deq = OQ.dequant(OQ.pack(fmt, W)).T.copy()
    for tile in range(1, wq.GEMM_TILES + 1):
        assert np.array_equal(_run_gemm(wq, g, synth.identity_activation(K), tile), _selected(fmt, tile, deq)), \
            f"gemm tile={tile}"


@pytest.mark.parametrize("fmt", ["w8g128", "w4g128"])
def test_gemm_fp16_activations_fall_back_to_exact(wq, fmt):
    """The group-128 LDS-DMA GEMM multiplies fp16 copies of x: a workgroup whose x holds
    a value fp16 cannot hold exactly (|x| > 65280, or 0 < |x| < 2^-17) recomputes its
    tile on the exact bf16 path; other workgroups stay on the fp16 path, and 40000 (fp16
    holds it) stays there too.  Huge weights (scales beyond fp16's range of products)
    change nothing: codes stay exact and scales multiply fp32 sums."""
    K, N, M = 1024, 520, 300   # three 128-row blocks of x, three 256-column blocks
    W = synth.weight(105, K, N, synth.uses_outliers(fmt))
    W[300:308] *= np.float32(1.5e5 if fmt == "w4g128" else 2.0e6)  # huge weights in one 8-row block
    g, can = quantize_on_gpu(wq, W, fmt)
    P = OQ.pack(fmt, W)
    sc = np.abs(P["scales"].astype(np.float32) if fmt == "w4g128" else OQ.bf16_bits_to_f32(P["scales"]))
    assert sc.max() > (4096 if fmt == "w4g128" else 512) and np.isfinite(sc).all()
    xf = OQ.bf16_bits_to_f32(synth.activation(105, K, M)).copy()
    for case in ("plain", "big-x", "tiny-x"):
        if case == "big-x":
            xf[5, 17] = 40000.0                 # fp16 holds it: the first row block stays on fp16
            xf[6, 900] = -3.0e5                 # beyond fp16: the first row block falls back
        if case == "tiny-x":
            xf[200, 33] = 3.0e-7                # below 2^-17: the second row block falls back
        x = OQ.bf16_rne_bits(xf.astype(np.float32))
        y_ref = OL.ref_linear(x, P)
        for tile in (9, 11, 13, 15, 18, 1):   # 11: split-K (fp32 partials, also on the exact path); 15, 18: 64- and 128-row tiles
            assert_parity(_run_gemm(wq, g, x, tile), y_ref, f"{fmt} {case} tile={tile}")
        # without a workspace tile 9 converts x to fp16 inside each workgroup: same bits
        assert np.array_equal(_run_gemm(wq, g, x, 9, with_ws=False), _run_gemm(wq, g, x, 9)), f"{fmt} {case}"


@pytest.mark.parametrize("fmt", OQ.FORMATS)
def test_zero_and_power_of_two_scaling(wq, fmt):
    """x = 0 gives y = 0; x * 4 gives y * 4 bit-exactly.  The scaling invariant
    holds when no intermediate is subnormal, so x is kept at |x| >= 2^-8 (the int8
    path carries x as fp16, whose subnormals start below 2^-14)."""
    K, N = 8192, 264
    W = synth.weight(96, K, N, synth.uses_outliers(fmt))
    g, can = quantize_on_gpu(wq, W, fmt)
    zero = np.zeros((3, K), dtype=np.uint16)
    assert not np.any(_run_gemv(wq, g, zero, 4) & 0x7FFF)
    assert not np.any(_run_gemm(wq, g, np.zeros((20, K), dtype=np.uint16)) & 0x7FFF)
    xf = OQ.bf16_bits_to_f32(synth.activation(96, K, 4))
    xf = np.where(np.abs(xf) < 2.0 ** -8, np.copysign(np.float32(2.0 ** -8), xf), xf).astype(np.float32)
    x = OQ.bf16_rne_bits(xf)
    x4 = OQ.bf16_rne_bits(OQ.bf16_bits_to_f32(x) * np.float32(4.0))
    for split in (1, 4):
        a = OQ.bf16_bits_to_f32(_run_gemv(wq, g, x, split))
        b = OQ.bf16_bits_to_f32(_run_gemv(wq, g, x4, split))
        assert np.array_equal(a * np.float32(4.0), b)


@pytest.mark.parametrize("fmt", OQ.FORMATS)
def test_gemv_with_large_and_tiny_activations(wq, fmt):
    """Slices holding an x that fp16 cannot hold exactly (|x| > 65280, or 0 < |x| <
    2^-17) take the bf16 path of the GEMV; values at the edges of the fp16-exact range
    stay on the fp16 path.  Every case within tolerance of the oracle."""
    K, N = 8192, 264
    W = synth.weight(104, K, N, synth.uses_outliers(fmt))
    g, can = quantize_on_gpu(wq, W, fmt)
    P = OQ.pack(fmt, W)
    xf = OQ.bf16_bits_to_f32(synth.activation(104, K, 4)).copy()
    xf[0, 17] = 3.0e5           # bf16 path, beyond fp16
    xf[1, 2100] = -65280.0      # fp16 path: the largest bf16 magnitude fp16 holds
    xf[2, 3000] = 2.0 ** -17    # fp16 path: the smallest magnitude fp16 holds exactly
    xf[2, 3001] = -3.0e-8       # bf16 path: below 2^-17
    xf[3, 4100] = 510.0
    xf[3, 6000] = -500.0
    x = OQ.bf16_rne_bits(xf.astype(np.float32))
    y_ref = OL.ref_linear(x, P)
    for split in _allowed_splits(fmt, K)[:3]:
        assert_parity(_run_gemv(wq, g, x, split), y_ref, f"{fmt} large-x split={split}")
    # the matrix-core GEMV takes the same switch per 128-group
    xd = to_dev_bf16(x)
    for rows in (16 | wq.GEMV_MFMA, 64 | wq.GEMV_MFMA):
        if wq.wq_gemv_max_waves(fmt, 4, rows) > 0:
            y = torch.empty((4, N), dtype=torch.bfloat16, device=DEV)
            wq.wq_gemv_ex(g, xd, y, 1, 4, rows, ws=None)
            torch.cuda.synchronize()
            assert_parity(bf16_bits(y), y_ref, f"{fmt} large-x rows={rows}")


def test_all_zero_rows_give_zero(wq):
    K, N = 4096, 264
    for fmt in OQ.FORMATS:
        W = synth.weight(97, K, N, synth.uses_outliers(fmt))
        W[10] = 0
        g, can = quantize_on_gpu(wq, W, fmt)
        x = synth.activation(97, K, 5)
        assert not np.any(_run_gemv(wq, g, x, 2)[:, 10] & 0x7FFF)
        assert not np.any(_run_gemm(wq, g, synth.activation(97, K, 40))[:, 10] & 0x7FFF)


def test_repeat_runs_are_bit_identical(wq):
    K, N = 5120, 7168
    W = synth.weight(98, K, N)
    g, _ = quantize_on_gpu(wq, W, "w8pc")
    x = synth.activation(98, K, 4)
    for split in (1, 2, 4):
        first = _run_gemv(wq, g, x, split)
        for _ in range(3):
            assert np.array_equal(_run_gemv(wq, g, x, split), first)


def test_dispatch_boundary_m7_m8(wq):
    """wq_linear takes the GEMV at M = 7 and the GEMM at M = 8; both paths agree
    with the oracle, and the GEMM also accepts M = 1..7."""
    K, N = 5120, 7168
    W = synth.weight(99, K, N)
    g, _ = quantize_on_gpu(wq, W, "w8pc")
    rows = sample_rows(N, 64)
    P = oracle_pack_rows("w8pc", W, rows)
    ws = wq.workspace(wq.wq_workspace_size(g, 7))
    for M in (7, 8):
        x = synth.activation(99, K, M)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
        wq.wq_linear(g, to_dev_bf16(x), y, ws=ws)
        torch.cuda.synchronize()
        y_ref = OL.ref_linear(x, P)
        assert_parity(bf16_bits(y)[:, rows], y_ref, f"linear M={M}")
        if M == 7:
            assert_parity(_run_gemm(wq, g, x)[:, rows], y_ref, "gemm M=7")


@pytest.mark.parametrize("fmt", OQ.FORMATS)
def test_gemm_tail_round_split(wq, fmt):
    """Tile 13: the tiles (256 x 256 for per-channel W8: 2 x 140; 128 x 256 for
    group-128: 3 x 94), ragged in M and N, leave 24 resp. 26 tiles for a last round on a
    256-CU device, which are split over K into 4 fp32 partials (their own block per
    range) and added by a second kernel; compared with the oracle everywhere, also with
    huge weights in a tail tile and an activation below fp16's exact range in the last
    row block (group-128: its tiles, tail tiles among them, fall back to the exact path,
    which writes those partials); the default tile without a workspace runs it as tile
    9."""
    K, M = 1024, 300
    tm, nb = (256, 140) if fmt == "w8pc" else (128, 94)
    N = 256 * nb - (40 if fmt == "w4g128" else 37)     # odd N: the reduction's per-element stores
    W = synth.weight(107, K, N, synth.uses_outliers(fmt))
    if fmt != "w8pc":
        W[N - 800:N - 792] *= np.float32(1.5e5 if fmt == "w4g128" else 2.0e6)
    g, _ = quantize_on_gpu(wq, W, fmt)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    total = -(-M // tm) * nb
    if total > cus and 2 * (total % cus) <= cus:   # 256 CUs: 24 / 26 tiles left, split 4
        r = total % cus
        assert wq.wq_workspace_size(g, M) >= min(4, cus // r) * r * tm * 256 * 4
    xf = OQ.bf16_bits_to_f32(synth.activation(107, K, M)).copy()
    xf[290, 100] = 3.0e-7
    x = OQ.bf16_rne_bits(xf.astype(np.float32))
    y_ref = OL.ref_linear(x, OQ.pack(fmt, W))
    # tile 0 picks 13 here; without a workspace it runs as tile 9, tile 13 itself refuses
    for tile, with_ws in ((13, True), (0, True), (0, False), (9, True)):
        assert_parity(_run_gemm(wq, g, x, tile, with_ws), y_ref, f"{fmt} tile={tile} ws={with_ws}")
    with pytest.raises(wq.WqError):
        _run_gemm(wq, g, x, 13, with_ws=False)


def test_no_writes_outside_y_and_workspace(wq):
    """Canary bytes around y and the workspace stay untouched (ragged N tile,
    split-K)."""
    K, N, M = 5120, 1000, 3
    W = synth.weight(100, K, N)
    g, _ = quantize_on_gpu(wq, W, "w8g128")
    x = to_dev_bf16(synth.activation(100, K, M))
    pad = 4096
    ybuf = torch.full((M * N + 2 * pad,), 12345, dtype=torch.int16, device=DEV)
    y = ybuf[pad:pad + M * N].view(torch.bfloat16)
    nws = wq.wq_workspace_size(g, M)
    wsbuf = torch.zeros(nws + 2 * pad, dtype=torch.uint8, device=DEV)
    wsbuf[:pad] = 0xAB
    wsbuf[pad + nws:] = 0xCD
    ws = wsbuf[pad:pad + nws]
    for split in (1, 2, 4):
        wq.wq_gemv(g, x, y, split_k=split, ws=ws)
    yg = torch.full((40 * N + 2 * pad,), 321, dtype=torch.int16, device=DEV)
    wq.wq_gemm(g, to_dev_bf16(synth.activation(100, K, 40)), yg[pad:pad + 40 * N].view(torch.bfloat16))
    torch.cuda.synchronize()
    assert torch.all(ybuf[:pad] == 12345) and torch.all(ybuf[pad + M * N:] == 12345)
    assert torch.all(wsbuf[:pad] == 0xAB) and torch.all(wsbuf[pad + nws:] == 0xCD)
    assert torch.all(yg[:pad] == 321) and torch.all(yg[pad + 40 * N:] == 321)
    # the LDS-DMA tiles at M = 300: split-K partials and x in fp16 stay inside the workspace
    Mg = 300
    ng = wq.wq_workspace_size(g, Mg)
    assert ng >= Mg * K * 2
    wsg = torch.zeros(ng + 2 * pad, dtype=torch.uint8, device=DEV)
    wsg[:pad] = 0xAB
    wsg[pad + ng:] = 0xCD
    ybig = torch.full((Mg * N + 2 * pad,), 321, dtype=torch.int16, device=DEV)
    for tile in (9, 10, 11, 12, 13, 14, 15, 16, 17, 18, 19, 24, 25, 26, 27, 28):
        wq.wq_gemm(g, to_dev_bf16(synth.activation(100, K, Mg)), ybig[pad:pad + Mg * N].view(torch.bfloat16),
                   tile=tile, ws=wsg[pad:pad + ng])
    torch.cuda.synchronize()
    assert torch.all(wsg[:pad] == 0xAB) and torch.all(wsg[pad + ng:] == 0xCD)
    assert torch.all(ybig[:pad] == 321) and torch.all(ybig[pad + Mg * N:] == 321)


def test_hip_graph_replay(wq):
    """wq_linear captured in a HIP graph replays correctly, repeatedly, with eager
    work and synchronisation between replays."""
    K, N = 5120, 7168
    W = synth.weight(101, K, N)
    g, _ = quantize_on_gpu(wq, W, "w8pc")
    xs = {M: to_dev_bf16(synth.activation(101, K, M)) for M in (1, 4, 64)}
    ys = {M: torch.empty((M, N), dtype=torch.bfloat16, device=DEV) for M in xs}
    ws = wq.workspace(wq.wq_workspace_size(g, 7))
    eager = {}
    for M in xs:
        wq.wq_linear(g, xs[M], ys[M], ws=ws)
    torch.cuda.synchronize()
    eager = {M: ys[M].clone() for M in xs}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            for M in xs:
                wq.wq_linear(g, xs[M], ys[M], ws=ws)
    torch.cuda.synchronize()
    for it in range(4):
        for M in xs:
            ys[M].fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for M in xs:
            assert torch.equal(ys[M], eager[M]), (it, M)


def test_tuner_runs_and_caches(wq, tmp_path):
    K, N = 5120, 7168
    W = synth.weight(102, K, N)
    g, _ = quantize_on_gpu(wq, W, "w8pc")
    copies = [g, g.clone(), g.clone()]
    x = to_dev_bf16(synth.activation(102, K, 1))
    y = torch.empty((1, N), dtype=torch.bfloat16, device=DEV)
    ws = wq.workspace(wq.wq_workspace_size(g, 1))
    chosen, lat = wq.wq_tune(copies, x, y, ws, warmup=5, iters=10)
    smax = wq.wq_gemv_max_split("w8pc", K)
    assert chosen in SPLITS and chosen <= smax
    assert all((v > 0) == (s <= smax) for s, v in zip(SPLITS, lat)), lat
    v = wq.wq_tune_cache_get("w8pc", K, N, 1, 0)
    assert v & 0xFF == chosen and 1 <= (v >> 8) & 0xFF <= 16 and (v >> 16) & 0xFF in wq.ROWS_GRID
    p = str(tmp_path / "cache.txt")
    wq.wq_tune_cache_save(p)
    assert f" 0 {K} {N} 1 0 {v}" in open(p).read()
    xg = to_dev_bf16(synth.activation(102, K, 64))
    yg = torch.empty((64, N), dtype=torch.bfloat16, device=DEV)
    wsg = wq.workspace(wq.wq_workspace_size(g, 64))
    tile, lat = wq.wq_tune(copies, xg, yg, wsg, warmup=2, iters=3)
    # every tile runs at M = 64 but the matrix-core GEMV tiles (at most 16 tokens): not run
    assert 1 <= tile <= wq.GEMM_TILES and tile not in wq.MMA_TILES, (tile, lat)
    assert all((v > 0) == (t not in wq.MMA_TILES) for t, v in enumerate(lat, 1)), lat
    assert wq.wq_tune_cache_get("w8pc", K, N, 64, wq.KIND_GEMM) == tile
    # without a workspace the split-K tiles cannot run and are skipped
    tile, lat = wq.wq_tune(copies, xg, yg, None, warmup=2, iters=3)
    split_tiles = list(range(5, 9)) + list(range(10, 13)) + [15, 16, 18, 19, 24, 25, 26, 27, 28]  # the split-K tiles (skinny, LDS-DMA)
    assert tile not in split_tiles, (tile, lat)
    skipped = set(split_tiles) | set(wq.MMA_TILES)
    assert all((v < 0) == (t in skipped) for t, v in enumerate(lat, start=1)), (tile, lat)
    # at 12 tokens the matrix-core GEMV tiles run (tile 23, split-K 2, only with a workspace)
    x12 = to_dev_bf16(synth.activation(102, K, 12))
    y12 = torch.empty((12, N), dtype=torch.bfloat16, device=DEV)
    ws12 = wq.workspace(wq.wq_workspace_size(g, 12))
    tile, lat = wq.wq_tune(copies, x12, y12, ws12, warmup=2, iters=3)
    assert all(lat[t - 1] > 0 for t in wq.MMA_TILES), lat
    tile, lat = wq.wq_tune(copies, x12, y12, None, warmup=2, iters=3)
    assert lat[22] < 0 and all(lat[t - 1] > 0 for t in (20, 21, 22)), lat


def test_error_paths_on_device(wq):
    K, N = 9216, 264
    W = synth.weight(103, K, N)
    g, can = quantize_on_gpu(wq, W, "w8pc")
    x = to_dev_bf16(synth.activation(103, K, 2))
    y = torch.empty((2, N), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(wq.WqError) as e:
        wq.wq_gemv(can, x, y, split_k=1)              # canonical layout
    assert e.value.status == 2
    with pytest.raises(wq.WqError) as e:
        wq.wq_gemv(g, x, y, split_k=8, ws=torch.zeros(64, dtype=torch.uint8, device=DEV))
    assert e.value.status == 4
    # untuned split with no workspace falls back to one slice and still computes
    wq.wq_tune_cache_clear()
    wq.wq_linear(g, x, y)
    torch.cuda.synchronize()
    assert_parity(bf16_bits(y), OL.ref_linear(synth.activation(103, K, 2), OQ.pack("w8pc", W)), "no-ws")
