"""Plant plausible mistakes in the oracle (on the CPU) and check that at least
one pin fails for each: a pin set that a dropped term, a wrong sign, a wrong
index or a transposed operand slips through would not be a pin."""
import numpy as np
import pytest

import math

import oracle.linear as OL
import oracle.moe as OM
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


def _mut_rel_rms_over_result(mp):
    orig = OL.compare

    def bad(y_bits, y_ref):                             # divides by ||y|| instead of ||y_ref||
        st = orig(y_bits, y_ref)
        y = OQ.bf16_bits_to_f32(y_bits).astype(np.float64)
        d = float(np.sqrt(np.sum(y * y)))
        st["rel_rms"] = float(np.sqrt(np.sum((y - y_ref) ** 2))) / d if d > 0 else 0.0
        return st
    mp.setattr(OL, "compare", bad)


def _mut_rel_rms_zero_reference_absolute(mp):
    orig = OL.compare

    def bad(y_bits, y_ref):                             # absolute RMS when the reference is 0
        st = orig(y_bits, y_ref)
        if not np.any(y_ref):
            y = OQ.bf16_bits_to_f32(y_bits).astype(np.float64)
            st["rel_rms"] = float(np.sqrt(np.mean(y * y)))
        return st
    mp.setattr(OL, "compare", bad)


def _mut_topk_rows_first_u(mp):
    orig = OT.sample_row
    first = []

    def bad(kept_bits, kept_idx, temperature, u):       # every row draws with row 0's u
        if not first:
            first.append(u)
        return orig(kept_bits, kept_idx, temperature, first[0])
    orig_ref = OT.ref_topk_sample

    def ref(logit_bits, k, temperature, u):
        first.clear()
        return orig_ref(logit_bits, k, temperature, u)
    mp.setattr(OT, "sample_row", bad)
    mp.setattr(OT, "ref_topk_sample", ref)


def _mut_topk_rows_shifted(mp):
    def bad(logit_bits, k, temperature, u):             # row m draws from row m-1's kept set
        L = np.asarray(logit_bits, dtype=np.uint16)
        M = L.shape[0]
        u = np.asarray(u, dtype=np.float64).ravel()
        idx = np.zeros((M, k), dtype=np.int64)
        bits = np.zeros((M, k), dtype=np.uint16)
        tok = np.zeros(M, dtype=np.int64)
        for m in range(M):
            idx[m], bits[m] = OT.topk_row(L[m], k)
        for m in range(M):
            j = (m - 1) % M
            tok[m] = OT.sample_row(bits[j], idx[j], temperature, float(u[m]))
        return idx, bits, tok
    mp.setattr(OT, "ref_topk_sample", bad)


def _mut_silu_sign(mp):
    mp.setattr(OM, "silu", lambda v: np.asarray(v, dtype=np.float64) / (1.0 + np.exp(np.asarray(v, dtype=np.float64))))


def _mut_silu_mul_swapped(mp):
    def bad(y):                                          # silu of the up half times the gate half
        y = np.asarray(y, dtype=np.float64)
        i = y.shape[-1] // 2
        return OM.silu(y[..., i:]) * y[..., :i]
    mp.setattr(OM, "silu_mul", bad)


def _mut_moe_rows_shifted(mp):
    orig = OM.ref_moe_linear

    def bad(x_bits, offsets, packed):                    # expert e takes the rows one further on
        off = np.asarray(offsets).copy()
        off[1:-1] = np.minimum(off[1:-1] + 1, off[-1])
        return orig(x_bits, off, packed)
    mp.setattr(OM, "ref_moe_linear", bad)


def _mut_moe_expert_index(mp):
    orig = OM.ref_moe_linear

    def bad(x_bits, offsets, packed):                    # rows of expert e meet expert e - 1
        return orig(x_bits, offsets, [packed[(e - 1) % len(packed)] for e in range(len(packed))])
    mp.setattr(OM, "ref_moe_linear", bad)


def _mut_w4pc_groups_of_128(mp):
    orig = OQ.quantize_w4

    def bad(W, G=OQ.GROUP):                              # "per channel" quantised per 128 k
        return orig(W, OQ.GROUP if G is None else G)
    mp.setattr(OQ, "quantize_w4", bad)


def _mut_w4pc_zeros_reversed(mp):
    orig = OQ.pack

    def bad(fmt, W):
        P = orig(fmt, W)
        if fmt == "w4pc":                                # the 8 zero-points of a word in reverse order
            z = OQ._unpack_nibbles_rows(np.asarray(P["zeros"]).reshape(1, -1)).reshape(-1, 8)[:, ::-1]
            P["zeros"] = OQ._pack_nibbles_rows(np.ascontiguousarray(z.reshape(1, -1))).reshape(-1)
        return P
    mp.setattr(OQ, "pack", bad)


def _mut_w4pc_dequant_row0_zero(mp):
    orig = OQ.dequant

    def bad(P, rows=None):
        if P["fmt"] != "w4pc":
            return orig(P, rows)
        q, s16, z = OQ.unpack_w4pc(P)                     # every row takes row 0's zero-point
        d = (q.astype(np.float32) - np.float32(z[0])) * s16.astype(np.float32)[:, None]
        return d if rows is None else d[np.asarray(rows)]
    mp.setattr(OQ, "dequant", bad)


def _mut_small_groups_quantised_per_128(mp):
    orig = OQ.pack

    def bad(fmt, W):                                     # the g32 / g64 formats quantised in 128s
        if fmt in OQ.SMALL_GROUPS:
            P = orig(fmt[:3] + "128", W)
            P["fmt"] = fmt
            G = OQ.GROUPED[fmt]
            r = 128 // G                                  # ... with the scales spread to their shape
            P["scales"] = np.repeat(P["scales"], r, axis=1)
            if "zeros" in P:
                P["zeros"] = np.repeat(P["zeros"], r, axis=0)
            return P
        return orig(fmt, W)
    mp.setattr(OQ, "pack", bad)


def _mut_small_group_zeros_not_transposed(mp):
    orig = OQ.pack

    def bad(fmt, W):
        P = orig(fmt, W)
        if fmt in ("w4g32", "w4g64"):                    # zero-points packed along K, not along N
            q, s16, z = OQ.quantize_w4(W, OQ.GROUPED[fmt])
            zp = np.zeros((z.shape[0], -(-z.shape[1] // 8) * 8), dtype=np.uint8)
            zp[:, :z.shape[1]] = z                        # each row's groups in one run of words
            P["zeros"] = np.resize(OQ._pack_nibbles_rows(zp).reshape(-1), np.asarray(P["zeros"]).shape)
        return P
    mp.setattr(OQ, "pack", bad)


def _mut_small_group_dequant_tiles_scales(mp):
    orig = OQ.dequant

    def bad(P, rows=None):
        if P["fmt"] not in OQ.SMALL_GROUPS or not P["fmt"].startswith("w8"):
            return orig(P, rows)
        q = P["qweight"].astype(np.float32)              # column k takes group k % (K/G), not k // G
        s = OQ.bf16_bits_to_f32(P["scales"])
        d = q * np.tile(s, (1, OQ.GROUPED[P["fmt"]]))
        return d if rows is None else d[np.asarray(rows)]
    mp.setattr(OQ, "dequant", bad)


def _mut_f16_read_as_bf16(mp):
    orig = OL._x64

    def bad(x_bits, act="bf16"):                         # fp16 activations decoded as bf16
        return orig(x_bits, "bf16")
    mp.setattr(OL, "_x64", bad)


def _mut_f16_decode_drops_subnormals(mp):
    orig = OL.f16_bits_to_f64

    def bad(bits):                                       # fp16 subnormals flushed to zero
        v = orig(bits)
        return np.where(np.abs(v) < 2.0 ** -14, 0.0, v)
    mp.setattr(OL, "f16_bits_to_f64", bad)


def _mut_residual_subtracted(mp):
    orig = OL.ref_linear

    def bad(x_bits, P, r_bits, act="bf16"):              # the residual taken away instead of added
        y = orig(x_bits, P, act=act)
        return y - OL._x64(np.asarray(r_bits, dtype=np.uint16).reshape(y.shape), act)
    mp.setattr(OL, "ref_linear_residual", bad)


def _mut_residual_transposed(mp):
    orig = OL.ref_linear

    def bad(x_bits, P, r_bits, act="bf16"):              # r read as [N, M]
        y = orig(x_bits, P, act=act)
        r = np.asarray(r_bits, dtype=np.uint16).reshape(-1)
        return y + OL._x64(r.reshape(y.shape[1], y.shape[0]).T, act)
    mp.setattr(OL, "ref_linear_residual", bad)


MUTATIONS = [_mut_round_half_away, _mut_fp32_scale, _mut_zero_sign, _mut_dequant_drops_zero,
             _mut_nibble_order, _mut_zeros_along_k, _mut_drop_tail_chunk, _mut_truncating_bf16,
             _mut_wrong_group_index, _mut_threshold, _mut_topk_ties_larger_index,
             _mut_topk_ascending, _mut_topk_nan_first, _mut_topk_signed_zero,
             _mut_sample_temperature_multiplies, _mut_sample_at_or_above, _mut_perm_inverse,
             _mut_perm_out_of_range_wraps, _mut_rel_rms_over_result,
             _mut_rel_rms_zero_reference_absolute, _mut_topk_rows_first_u, _mut_topk_rows_shifted,
             _mut_silu_sign, _mut_silu_mul_swapped, _mut_moe_rows_shifted, _mut_moe_expert_index,
             _mut_w4pc_groups_of_128, _mut_w4pc_zeros_reversed, _mut_w4pc_dequant_row0_zero,
             _mut_small_groups_quantised_per_128, _mut_small_group_zeros_not_transposed,
             _mut_small_group_dequant_tiles_scales, _mut_f16_read_as_bf16, _mut_f16_decode_drops_subnormals,
             _mut_residual_subtracted, _mut_residual_transposed]


@pytest.mark.parametrize("mut", MUTATIONS, ids=lambda f: f.__name__)
def test_planted_mistake_is_caught(mut, monkeypatch):
    mut(monkeypatch)
    with pytest.raises(Exception):
        pins.run_all_pins()
