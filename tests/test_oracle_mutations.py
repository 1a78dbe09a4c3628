"""Plant plausible mistakes in the oracle (on the CPU) and check that at least
one pin fails for each: a pin set that a dropped term, a wrong sign, a wrong
index or a transposed operand slips through would not be a pin."""
import numpy as np
import pytest

import math

import oracle.linear as OL
import oracle.quant as OQ
import oracle.topk as OT
import pins


def _half_away(v):
    return np.sign(v) * np.floor(np.abs(v) + 0.5)


def _mut_round_half_away(mp):
    orig = np.rint
    mp.setattr(OQ.np, "rint", _half_away, raising=True)
    return orig


def _mut_fp32_scale(mp):
    orig = OQ.quantize_w8

    def bad(W, G=None):
        W = np.ascontiguousarray(W, dtype=np.float32)
        N, K = W.shape
        G = K if G is None else G
        Wg = W.reshape(N, K // G, G)
        a = np.max(np.abs(Wg), axis=2)
        s32 = a / np.float32(127.0)
        sb = OQ.bf16_rne_bits(s32)
        q = np.zeros(Wg.shape, np.float32)
        nz = s32 != 0
        q[nz] = np.clip(np.rint(Wg[nz] / s32[nz][:, None]), -127, 127)   # unrounded scale
        return q.astype(np.int8).reshape(N, K), sb
    mp.setattr(OQ, "quantize_w8", bad)
    return orig


def _mut_zero_sign(mp):
    orig = OQ.quantize_w4g128

    def bad(W):
        q, s16, z = orig(W)
        s = s16.astype(np.float32)
        Wg = np.ascontiguousarray(W, np.float32).reshape(W.shape[0], -1, 128)
        lo = Wg.min(axis=2)
        nz = s != 0
        z2 = np.zeros_like(s)
        z2[nz] = np.clip(np.rint(lo[nz] / s[nz]), 0, 15)          # sign flipped
        q2 = np.zeros(Wg.shape, np.float32)
        q2[nz] = np.clip(np.rint(Wg[nz] / s[nz][:, None]) + z2[nz][:, None], 0, 15)
        return q2.astype(np.uint8).reshape(W.shape), s16, z2.astype(np.uint8)
    mp.setattr(OQ, "quantize_w4g128", bad)


def _mut_dequant_drops_zero(mp):
    orig = OQ.dequant

    def bad(P, rows=None):
        if P["fmt"] != "w4g128":
            return orig(P, rows)
        sel = slice(None) if rows is None else np.asarray(rows)
        q = OQ._unpack_nibbles_rows(P["qweight"][sel]).astype(np.float32)
        s = P["scales"][sel].astype(np.float32)
        n, K = q.shape
        return (q.reshape(n, K // 128, 128) * s[:, :, None]).reshape(n, K)   # no "- z"
    mp.setattr(OQ, "dequant", bad)


def _mut_nibble_order(mp):
    def bad(v):
        R, L = v.shape
        v = v.astype(np.uint32).reshape(R, L // 8, 8)
        out = np.zeros((R, L // 8), dtype=np.uint32)
        for j in range(8):
            out |= v[:, :, j] << np.uint32(4 * (7 - j))                    # high nibble first
        return out
    mp.setattr(OQ, "_pack_nibbles_rows", bad)


def _mut_zeros_along_k(mp):
    orig = OQ.pack

    def bad(fmt, W):
        P = orig(fmt, W)
        if fmt == "w4g128":
            q, s16, z = OQ.quantize_w4g128(W)
            P["zeros"] = np.ascontiguousarray(OQ._pack_nibbles_rows(
                np.pad(z, ((0, 0), (0, (-z.shape[1]) % 8)))).T)               # packed along K
        return P
    mp.setattr(OQ, "pack", bad)


def _mut_drop_tail_chunk(mp):
    def bad(x_bits, P, chunk=4096):
        x = OQ.bf16_bits_to_f32(x_bits).astype(np.float64)
        N = P["N"]
        y = np.zeros((x.shape[0], N))
        for n0 in range(0, N - chunk + 1, chunk):                           # drops the tail
            rows = np.arange(n0, n0 + chunk)
            y[:, n0:n0 + chunk] = x @ OQ.dequant(P, rows).astype(np.float64).T
        return y
    mp.setattr(OL, "ref_linear", bad)


def _mut_truncating_bf16(mp):
    def bad(a):
        u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
        return (u >> np.uint32(16)).astype(np.uint16)
    mp.setattr(OQ, "bf16_rne_bits", bad)


def _mut_wrong_group_index(mp):
    orig = OQ.dequant

    def bad(P, rows=None):
        if P["fmt"] != "w8g128":
            return orig(P, rows)
        sel = slice(None) if rows is None else np.asarray(rows)
        q = P["qweight"][sel].astype(np.float32)
        s = OQ.bf16_bits_to_f32(P["scales"][sel])
        n, K = q.shape
        return (q.reshape(n, 128, K // 128) * s[:, None, :]).reshape(n, K)   # groups strided
    mp.setattr(OQ, "dequant", bad)


def _mut_threshold(mp):
    mp.setattr(OL, "use_gemv", lambda M: M <= 8)


def _mut_topk_ties_larger_index(mp):
    mp.setattr(OT, "_rank_key", lambda v, i: (1, 0.0, -i) if math.isnan(v) else (0, -v, -i))


def _mut_topk_ascending(mp):
    mp.setattr(OT, "_rank_key", lambda v, i: (1, 0.0, i) if math.isnan(v) else (0, v, i))


def _mut_topk_nan_first(mp):
    mp.setattr(OT, "_rank_key", lambda v, i: (-1, 0.0, i) if math.isnan(v) else (0, -v, i))


def _mut_topk_signed_zero(mp):
    def key(v, i):
        if math.isnan(v):
            return (1, 0.0, i)
        if v == 0 and math.copysign(1.0, v) < 0:
            return (0, 1e-300, i)                       # -0 ranked below +0
        return (0, -v, i)
    mp.setattr(OT, "_rank_key", key)


def _mut_sample_temperature_multiplies(mp):
    mp.setattr(OT, "_weight", lambda v, v1, T: math.exp((v - v1) * T))


def _mut_sample_at_or_above(mp):
    mp.setattr(OT, "_reached", lambda run, u: run >= u)


def _mut_perm_inverse(mp):
    orig = OL.gather_activations

    def bad(x_bits, perm):                              # x'[perm[j]] = x[j]: the inverse gather
        perm = np.asarray(perm)
        inv = np.full(perm.size, perm.size, dtype=np.int64)
        ok = (perm >= 0) & (perm < perm.size)
        inv[perm[ok]] = np.nonzero(ok)[0]
        return orig(x_bits, inv)
    mp.setattr(OL, "gather_activations", bad)


def _mut_perm_out_of_range_wraps(mp):
    orig = OL.gather_activations
    mp.setattr(OL, "gather_activations", lambda x_bits, perm: orig(x_bits, np.asarray(perm) % np.asarray(x_bits).shape[-1]))


MUTATIONS = [_mut_round_half_away, _mut_fp32_scale, _mut_zero_sign, _mut_dequant_drops_zero,
             _mut_nibble_order, _mut_zeros_along_k, _mut_drop_tail_chunk, _mut_truncating_bf16,
             _mut_wrong_group_index, _mut_threshold, _mut_topk_ties_larger_index,
             _mut_topk_ascending, _mut_topk_nan_first, _mut_topk_signed_zero,
             _mut_sample_temperature_multiplies, _mut_sample_at_or_above, _mut_perm_inverse,
             _mut_perm_out_of_range_wraps]


@pytest.mark.parametrize("mut", MUTATIONS, ids=lambda f: f.__name__)
def test_planted_mistake_is_caught(mut, monkeypatch):
    mut(monkeypatch)
    with pytest.raises(Exception):
        pins.run_all_pins()
