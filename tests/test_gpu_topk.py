"""LM head + top-k sampling through the C ABI against the oracle.

The oracle computes its own logits (fp64, rounded to bf16), their top-k and the
drawn token.  Logits that differ from the oracle's within the layer's tolerance can
swap places with a neighbour whose value is as close, so the kept set is compared
where it is unique: every kept entry matches the oracle's logit within tolerance,
beats every dropped entry up to twice the tolerance, and the order and the ties
follow the stated rule on the kernel's own values.  Draws use a u in the middle of
the oracle's widest probability interval, so that the token is decided away from
any boundary; they are compared when the kept sets agree, and on every row against the
oracle's draw over the layer's own kept logits with the same u (unless u falls within
1e-4 of one of that distribution's boundaries).  The same order is also checked
exactly against the logits the layer itself returns (wq_linear)."""
import numpy as np
import pytest
import torch

import oracle.linear as OL
import oracle.quant as OQ
import oracle.topk as OT
import synth
from gpu_util import (DEV, bf16_bits, host_weight, oracle_pack_rows, quantize_on_gpu, sample_rows,
                      to_dev_bf16)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wq(wqlib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return wqlib


def _run(wq, g, x_bits, k, T, u):
    M = x_bits.shape[0]
    ws = wq.workspace(wq.wq_lm_head_topk_workspace_size(g, M, k))
    vals = torch.empty((M, k), dtype=torch.bfloat16, device=DEV)
    idx = torch.empty((M, k), dtype=torch.int32, device=DEV)
    tok = torch.empty(M, dtype=torch.int32, device=DEV)
    ud = torch.tensor(np.asarray(u, np.float32), device=DEV)
    wq.wq_lm_head_topk(g, to_dev_bf16(x_bits), k, T, ud, vals, idx, tok, ws)
    torch.cuda.synchronize()
    return bf16_bits(vals), idx.cpu().numpy().astype(np.int64), tok.cpu().numpy().astype(np.int64)


def _layer_logits(wq, g, x_bits):
    M = x_bits.shape[0]
    y = torch.empty((M, g.N), dtype=torch.bfloat16, device=DEV)
    ws = wq.workspace(wq.wq_workspace_size(g, M))
    wq.wq_linear(g, to_dev_bf16(x_bits), y, ws=ws)
    torch.cuda.synchronize()
    return bf16_bits(y)


def _order_of(bits_row):
    """The stated order on one row of bf16 bits (NaN-free), by a NumPy lexsort: larger
    value first, then smaller index; -0 and +0 compare equal as floats."""
    v = OQ.bf16_bits_to_f32(bits_row).astype(np.float64)
    return np.lexsort((np.arange(v.size), -v))


def _mid_u(bits_kept, T):
    """u in the middle of the widest interval of the oracle's draw distribution."""
    if T == 0:
        return 0.5
    v = OQ.bf16_bits_to_f32(bits_kept).astype(np.float64)
    p = np.exp((v - v[0]) / T)
    c = np.cumsum(p / p.sum())
    lo = np.concatenate([[0.0], c[:-1]])
    j = int(np.argmax(c - lo))
    return float((lo[j] + c[j]) / 2)


def _near_boundary(bits_kept, T, u, margin=1e-4):
    """Whether u lies within `margin` of a running-sum boundary of the draw over these
    kept logits (fp64): there fp32 arithmetic may legitimately pick the neighbour."""
    if T == 0:
        return False
    v = OQ.bf16_bits_to_f32(bits_kept).astype(np.float64)
    p = np.exp((v - v[0]) / T)
    c = np.cumsum(p / p.sum())
    return bool(np.min(np.abs(c - u)) < margin)


def _check_row(name, got_vals, got_idx, got_tok, y_ref_row, k, T, u, ref_idx, ref_tok):
    tol = OL.TOL_REL * np.maximum(1.0, np.abs(y_ref_row))
    assert len(set(got_idx.tolist())) == k, name
    # kept values are the logits at the kept indices, within the layer's tolerance
    gv = OQ.bf16_bits_to_f32(got_vals).astype(np.float64)
    assert np.all(np.abs(gv - y_ref_row[got_idx]) <= tol[got_idx] + np.abs(y_ref_row[got_idx]) * 2.0 ** -8), name
    # the kernel's own order on its values: non-increasing, equal values by index
    assert np.all((gv[:-1] > gv[1:]) | ((gv[:-1] == gv[1:]) & (got_idx[:-1] < got_idx[1:]))), name
    # the kept set beats the dropped one up to twice the tolerance
    kept = np.zeros(y_ref_row.size, bool)
    kept[got_idx] = True
    worst_kept = np.min(y_ref_row[kept] + 2 * tol[kept])
    assert np.all(y_ref_row[~kept] - 2 * tol[~kept] <= worst_kept), name
    assert got_tok in set(got_idx.tolist()), name
    if set(got_idx.tolist()) == set(ref_idx.tolist()):
        assert got_tok == ref_tok, (name, got_tok, ref_tok)


CASES = [("w8pc", 256, 5000, 1), ("w8g128", 256, 4100, 3), ("w4g128", 256, 6000, 7),
         ("w8pc", 384, 2047, 8), ("w4g128", 128, 9000, 2)]


@pytest.mark.parametrize("fmt,K,V,M", CASES)
def test_topk_against_oracle(wq, fmt, K, V, M):
    """Ragged vocabularies (one to five 2048-logit chunks), GEMV and GEMM (M = 8)
    logits, k from 1 to 64, greedy and two temperatures."""
    W = synth.weight(201, K, V, synth.uses_outliers(fmt)) * np.float32(20.0)   # logits ~ N(0, 6^2)
    g, _ = quantize_on_gpu(wq, W, fmt)
    P = OQ.pack(fmt, W)
    x = synth.activation(201, K, M)
    y_ref = OL.ref_linear(x, P)
    ref_bits = OQ.bf16_rne_bits(y_ref.astype(np.float32))
    own = _layer_logits(wq, g, x)
    for k in (1, 5, 64):
        for T in (0.0, 0.7, 2.0):
            u = []
            for m in range(M):
                ridx, rbits = OT.topk_row(ref_bits[m], k)
                u.append(_mid_u(rbits, T))
            ref_idx, ref_kb, ref_tok = OT.ref_topk_sample(ref_bits, k, T, u)
            vals, idx, tok = _run(wq, g, x, k, T, u)
            for m in range(M):
                name = f"{fmt} K={K} V={V} M={M} m={m} k={k} T={T}"
                _check_row(name, vals[m], idx[m], tok[m], y_ref[m], k, T, u[m], ref_idx[m], ref_tok[m])
                # exactly the stated order on the layer's own logits
                want = _order_of(own[m])[:k]
                assert np.array_equal(idx[m], want), name
                assert np.array_equal(vals[m], own[m][want]), name
                # the token against the oracle's draw on those same kept logits, whether or
                # not the kept set matches the oracle's own (u away from a boundary)
                if not _near_boundary(own[m][want], T, u[m]):
                    assert tok[m] == OT.sample_row(own[m][want], want, T, u[m]), name
                if T == 0:
                    assert tok[m] == idx[m][0], name


def test_topk_chunks_with_equal_tops(wq):
    """Weight rows repeating every 2048 rows give every 2048-logit chunk the same values,
    so each chunk's k best tie with every other chunk's and the merge must order equal
    values across chunks by index (ten chunks at k = 64 and 7, five at k = 64).  Order
    and token exactly as stated on the layer's own logits."""
    K = 128
    base = synth.weight(203, K, 2048) * np.float32(20.0)
    for chunks, k in ((10, 64), (5, 64), (10, 7)):
        V = 2048 * chunks
        W = np.tile(base, (chunks, 1))
        g, _ = quantize_on_gpu(wq, W, "w8pc")
        x = synth.activation(203, K, 2)
        own = _layer_logits(wq, g, x)
        for T in (0.0, 1.0):
            u = [0.31, 0.77]
            vals, idx, tok = _run(wq, g, x, k, T, u)
            for m in range(2):
                name = f"equal tops chunks={chunks} k={k} T={T} m={m}"
                want = _order_of(own[m])[:k]
                assert np.array_equal(idx[m], want), name
                assert np.array_equal(vals[m], own[m][want]), name
                if not _near_boundary(own[m][want], T, u[m]):
                    assert tok[m] == OT.sample_row(own[m][want], want, T, u[m]), name


def test_topk_ties_signed_zeros_and_repeat(wq):
    """All-zero weights give logits that are all +0 or -0: every entry ties, so the k
    smallest indices are kept and any draw at T > 0 is uniform over them; the call is
    bit-identical from run to run and under HIP graph replay."""
    K, V, M, k = 128, 3000, 2, 16
    W = np.zeros((V, K), np.float32)
    g, _ = quantize_on_gpu(wq, W, "w8pc")
    x = synth.activation(202, K, M)
    u = [0.0, 0.999]
    vals, idx, tok = _run(wq, g, x, k, 1.0, u)
    for m in range(M):
        assert idx[m].tolist() == list(range(k))
        assert np.all((vals[m] & 0x7FFF) == 0)
    assert tok.tolist() == [0, k - 1]                  # u = 0 -> first, u = 0.999 -> last
    # u = (j + 1/2) / k -> the (j+1)-th kept token
    for j in (3, 9):
        _, _, t2 = _run(wq, g, x, k, 1.0, [(j + 0.5) / k] * M)
        assert t2.tolist() == [j] * M
    # run-to-run and graph replay
    W2 = synth.weight(203, K, V) * np.float32(20.0)
    g2, _ = quantize_on_gpu(wq, W2, "w4g128")
    ws = wq.workspace(wq.wq_lm_head_topk_workspace_size(g2, M, k))
    xd = to_dev_bf16(synth.activation(203, K, M))
    ud = torch.tensor([0.3, 0.8], dtype=torch.float32, device=DEV)
    outs = [torch.empty((M, k), dtype=torch.bfloat16, device=DEV), torch.empty((M, k), dtype=torch.int32, device=DEV),
            torch.empty(M, dtype=torch.int32, device=DEV)]

    def call():
        wq.wq_lm_head_topk(g2, xd, k, 0.9, ud, *outs, ws)

    call()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr, stream=s):
            call()
    for _ in range(3):
        for o in outs:
            o.zero_()
        gr.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, eager):
            assert torch.equal(a, b)
        call()                                         # eager work between replays
        torch.cuda.synchronize()


LM_HEAD = [(4, "w8g128", 5120, 151936), (4, "w4g128", 5120, 151936), (4, "w8pc", 5120, 151936)]


@pytest.mark.parametrize("cfg,fmt,K,V", LM_HEAD)
def test_topk_full_lm_head(wq, cfg, fmt, K, V):
    """The LM-head shape (74 chunks): the kept logits against the oracle's at the
    kept rows, the order exactly against the layer's own logits, and no sampled
    row of the oracle beats the kept set beyond twice the tolerance."""
    W = host_weight(cfg, K, V, synth.uses_outliers(fmt))
    g, _ = quantize_on_gpu(wq, W, fmt)
    k, T = 50, 0.8
    for M in (1, 4):
        x = synth.activation(cfg, K, M)
        u = [0.37 + 0.1 * m for m in range(M)]
        vals, idx, tok = _run(wq, g, x, k, T, u)
        own = _layer_logits(wq, g, x)
        rows = np.unique(np.concatenate([sample_rows(V, 64, seed=cfg)] +
                                        [np.arange(8 * (i // 8), 8 * (i // 8) + 8) for i in idx.ravel()]))
        P = oracle_pack_rows(fmt, W, rows)
        y_rows = OL.ref_linear(x, P)                      # oracle logits at `rows`
        pos = {int(r): j for j, r in enumerate(rows)}
        for m in range(M):
            name = f"{fmt} M={M} m={m}"
            want = _order_of(own[m])[:k]
            assert np.array_equal(idx[m], want), name
            assert np.array_equal(vals[m], own[m][want]), name
            assert tok[m] in set(idx[m].tolist()), name
            if not _near_boundary(own[m][want], T, u[m]):   # the oracle's draw on these kept logits
                assert tok[m] == OT.sample_row(own[m][want], want, T, u[m]), name
            ref_kept = np.array([y_rows[m, pos[int(i)]] for i in idx[m]])
            tol_k = OL.TOL_REL * np.maximum(1.0, np.abs(ref_kept))
            gv = OQ.bf16_bits_to_f32(vals[m]).astype(np.float64)
            assert np.all(np.abs(gv - ref_kept) <= tol_k + np.abs(ref_kept) * 2.0 ** -8), name
            others = np.array([pos[int(r)] for r in rows if int(r) not in set(idx[m].tolist())])
            yo = y_rows[m, others]
            tol_o = OL.TOL_REL * np.maximum(1.0, np.abs(yo))
            assert np.all(yo - 2 * tol_o <= np.min(ref_kept + 2 * tol_k)), name
