"""Pins of the CPU oracle to facts other than itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with a
hand-derived worked example (tests/golden/), a closed-form bound, a brute-force
computation on tiny inputs written independently of the oracle (Python ints and
Fractions), or a reduction to a NumPy library routine.  The functions call the
oracle through its modules (``oracle.quant.X``, ``oracle.linear.X``) so that the
mutation tests can plant a mistake in the oracle and check that a pin fails.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

import oracle.linear as OL
import oracle.moe as OM
import oracle.quant as OQ
import oracle.topk as OT
import synth
from golden_io import num, read_fixture


# ------------------------------------------------------------ independent helpers
def _f32_fraction(v) -> Fraction:
    return Fraction(float(np.float32(v)))


def _bf16_bits_value(b: int) -> Fraction:
    """Exact value of a bf16 bit pattern, decoded by hand (normal and zero only)."""
    sign = -1 if b & 0x8000 else 1
    e = (b >> 7) & 0xFF
    m = b & 0x7F
    if e == 0:
        return Fraction(sign * m, 2 ** (126 + 7))
    return sign * Fraction(128 + m, 128) * Fraction(2) ** (e - 127)


def _fp16_value(h) -> Fraction:
    b = int(np.asarray(h, dtype=np.float16).view(np.uint16))
    sign = -1 if b & 0x8000 else 1
    e = (b >> 10) & 0x1F
    m = b & 0x3FF
    if e == 0:
        return Fraction(sign * m, 2 ** 24)
    return sign * Fraction(1024 + m, 1024) * Fraction(2) ** (e - 15)


def _decode_w4_codes(P: dict, n: int, k: int) -> int:
    word = int(P["qweight"][n, k // 8])
    return (word >> (4 * (k % 8))) & 0xF


def _decode_w4_zero(P: dict, n: int, g: int) -> int:
    word = int(P["zeros"][g, n // 8])
    return (word >> (4 * (n % 8))) & 0xF


def _decode_w4pc_zero(P: dict, n: int) -> int:
    word = int(np.asarray(P["zeros"]).reshape(-1)[n // 8])
    return (word >> (4 * (n % 8))) & 0xF


def _group_of(fmt: str) -> int:
    """Group size spelled in a grouped format's name (w8g32 -> 32, w4g128 -> 128)."""
    return int(fmt[3:])


def _exact_dequant(P: dict, n: int, k: int) -> Fraction:
    fmt = P["fmt"]
    if fmt == "w4pc":
        return (_decode_w4_codes(P, n, k) - _decode_w4pc_zero(P, n)) * _fp16_value(P["scales"][n])
    if fmt == "w8pc":
        return int(P["qweight"][n, k]) * _bf16_bits_value(int(P["scales"][n]))
    g = k // _group_of(fmt)
    if fmt.startswith("w8g"):
        return int(P["qweight"][n, k]) * _bf16_bits_value(int(P["scales"][n, g]))
    q = _decode_w4_codes(P, n, k)
    z = _decode_w4_zero(P, n, g)
    return (q - z) * _fp16_value(P["scales"][n, g])


# ------------------------------------------------------------------ conversions
def pin_bf16_rounding():
    """bf16 RNE: hand values, then brute force: the result is the nearer of the
    two bf16 neighbours of v (ties to the even one)."""
    f = OQ.bf16_rne_bits
    hand = {1.0: 0x3F80, 1.0 + 2 ** -8: 0x3F80, 1.0 + 3 * 2 ** -8: 0x3F82,
            -2.0: 0xC000, 0.0: 0x0000, 1.0 / 127.0: 0x3C01, 2.0 ** -7: 0x3C00,
            1.0 + 2 ** -8 + 2 ** -20: 0x3F81}
    for v, b in hand.items():
        got = int(f(np.array([v], dtype=np.float32))[0])
        assert got == b, f"bf16({v!r}) = {got:#06x}, expected {b:#06x}"
    rng = np.random.default_rng(123)
    vals = (rng.standard_normal(4000) * np.exp(rng.uniform(-20, 20, 4000))).astype(np.float32)
    bits = f(vals)
    for v, b in zip(vals[:800], bits[:800]):
        exact = _f32_fraction(v)
        u = int(np.float32(v).view(np.uint32))
        lo, hi = u >> 16, (u >> 16) + 1
        dlo = abs(_bf16_bits_value(lo) - exact)
        dhi = abs(_bf16_bits_value(hi) - exact)
        want = lo if dlo < dhi else hi if dhi < dlo else (lo if lo % 2 == 0 else hi)
        assert int(b) == want, f"bf16 rounding of {v!r}: {int(b):#x} vs {want:#x}"
    back = OQ.bf16_bits_to_f32(np.array([0x3F80, 0xC000, 0x3C01], dtype=np.uint16))
    assert [_f32_fraction(v) for v in back] == [1, -2, Fraction(129, 16384)]


# ------------------------------------------------------------------- quantisers
def pin_golden_w8pc():
    head, blk = read_fixture("w8pc_worked.txt")
    K, N = int(head["K"][0]), int(head["N"][0])
    W = np.array([[float(t) for t in r] for r in blk["W"]], dtype=np.float32)
    assert W.shape == (N, K)
    P = OQ.pack("w8pc", W)
    q = np.array([[int(float(t)) for t in r] for r in blk["q"]])
    s = np.array([num(r[0]) for r in blk["s_bits"]])
    assert np.array_equal(P["qweight"].astype(int), q), (P["qweight"], q)
    assert np.array_equal(P["scales"].astype(int), s), (P["scales"], s)
    assert P["qweight"].dtype == np.int8 and P["scales"].dtype == np.uint16


def _golden_w4_weight():
    head, _ = read_fixture("w4g128_worked.txt")
    K = int(head["K"][0])
    W = np.zeros((8, K), dtype=np.float32)    # N = 8 (zeros pack 8 per word); rows 1..7 zero
    exp_q = np.zeros((8, K), dtype=int)
    exp_s, exp_z = [], []
    for g in range(2):
        vals = [float(t) for t in head[f"group{g}"]]
        fill = float(head[f"group{g}_fill"][0])
        row = np.full(128, fill, dtype=np.float32)
        row[:len(vals)] = vals
        W[0, 128 * g:128 * (g + 1)] = row
        qv = [int(t) for t in head[f"group{g}_q"]]
        qrow = np.full(128, int(head[f"group{g}_fill_q"][0]))
        qrow[:len(qv)] = qv
        exp_q[0, 128 * g:128 * (g + 1)] = qrow
        exp_s.append(num(head[f"group{g}_s_bits"][0]))
        exp_z.append(int(head[f"group{g}_z"][0]))
    return W, exp_q, exp_s, exp_z


def pin_golden_w4g128():
    W, exp_q, exp_s, exp_z = _golden_w4_weight()
    P = OQ.pack("w4g128", W)
    for k in range(W.shape[1]):
        assert _decode_w4_codes(P, 0, k) == exp_q[0, k], f"q[0,{k}]"
    sbits = P["scales"].view(np.uint16)
    assert [int(sbits[0, g]) for g in range(2)] == exp_s, sbits[0]
    assert [_decode_w4_zero(P, 0, g) for g in range(2)] == exp_z
    # all-zero rows 1..7: scale 0, zero-point 0, codes 0 (every code equals its zero-point)
    assert not np.any(sbits[1:]) and all(_decode_w4_zero(P, n, g) == 0 for n in range(1, 8) for g in range(2))
    # dequantised row 0 equals (q - z) * s exactly
    Wd = OQ.dequant(P)
    for k in range(0, W.shape[1], 7):
        assert Fraction(float(Wd[0, k])) == _exact_dequant(P, 0, k)
    assert not np.any(Wd[1:])


def pin_golden_w4pc():
    """The per-channel W4 quantiser and its canonical packing against the hand-derived
    rows of tests/golden/w4pc_worked.txt: ties in both directions, an all-zero row, a
    constant row, a clamped zero-point, clamped codes, an fp16-rounded scale, and an
    odd zero-point where adding z before rounding would differ."""
    head, blocks = read_fixture("w4pc_worked.txt")
    W = np.array([[float(t) for t in r] for r in blocks["W"]], dtype=np.float32)
    exp_q = [[int(t) for t in r] for r in blocks["q"]]
    P = OQ.pack("w4pc", W)
    N, K = W.shape
    for n in range(N):
        assert [_decode_w4_codes(P, n, k) for k in range(K)] == exp_q[n], f"q row {n}"
    assert [int(w) for w in P["qweight"][:, 0]] == [num(t) for t in head["qweight_words"]]
    assert [int(b) for b in np.asarray(P["scales"]).view(np.uint16)] == [num(t) for t in head["s_bits"]]
    assert [_decode_w4pc_zero(P, n) for n in range(N)] == [int(t) for t in head["z"]]
    assert int(np.asarray(P["zeros"]).reshape(-1)[0]) == num(head["zeros_word"][0])
    Wd = OQ.dequant(P)
    for n in range(N):
        for k in range(K):
            assert Fraction(float(Wd[n, k])) == _exact_dequant(P, n, k), (n, k)
    assert not np.any(Wd[1]) and not np.any(Wd[2])


def pin_w4pc_one_group_is_group128(seed=12, N=24):
    """With K = 128 a per-channel group is exactly one group of 128: the two formats
    store the same codes, scales and zero-points (laid out as their layouts say)."""
    W = synth.weight(seed, 128, N, outliers=True)
    Pc, Pg = OQ.pack("w4pc", W), OQ.pack("w4g128", W)
    assert np.array_equal(Pc["qweight"], Pg["qweight"])
    assert np.array_equal(np.asarray(Pc["scales"]).view(np.uint16), np.asarray(Pg["scales"]).view(np.uint16)[:, 0])
    assert np.array_equal(np.asarray(Pc["zeros"]).reshape(-1), np.asarray(Pg["zeros"])[0])
    assert np.array_equal(OQ.dequant(Pc), OQ.dequant(Pg))


def pin_w4pc_roundtrip_bound(seed=13, N=32, K=1024):
    """P2 for one group per row: unclamped codes within s/2 of w, clamped ones within
    s/2 + (hi - lo) 2^-11; the scale comes from the whole row's range."""
    W = synth.weight(seed, K, N, outliers=True)
    P = OQ.pack("w4pc", W)
    s = np.asarray(P["scales"]).astype(np.float64)
    span = W.max(axis=1).astype(np.float64) - W.min(axis=1).astype(np.float64)
    for n in range(N):
        assert abs(float(s[n]) - span[n] / 15) <= span[n] / 15 * 2.0 ** -10, n
        z = _decode_w4pc_zero(P, n)
        for k in range(0, K, 7):
            wd = (_decode_w4_codes(P, n, k) - z) * float(s[n])
            assert abs(float(W[n, k]) - wd) <= s[n] / 2 + span[n] * 2.0 ** -11 + abs(float(W[n, k])) * 2.0 ** -22, (n, k)


def pin_golden_small_groups():
    """Groups of 32 and 64 against tests/golden/small_groups_worked.txt: groups built
    from the hand-derived per-channel rows, repeated, take those rows' codes, scales
    and zero-points, group by group, in the canonical layout."""
    head, _ = read_fixture("small_groups_worked.txt")
    _, b4 = read_fixture("w4pc_worked.txt")
    h4, _ = read_fixture("w4pc_worked.txt")
    W4 = np.array([[float(t) for t in r] for r in b4["W"]], dtype=np.float32)
    q4 = [[int(t) for t in r] for r in b4["q"]]
    s4 = [num(t) for t in h4["s_bits"]]
    z4 = [int(t) for t in h4["z"]]
    _, b8 = read_fixture("w8pc_worked.txt")
    W8 = np.array([[float(t) for t in r] for r in b8["W"]], dtype=np.float32)
    q8 = [[int(float(t)) for t in r] for r in b8["q"]]
    s8 = [num(r[0]) for r in b8["s_bits"]]
    for G in (32, 64):
        rep = G // 8
        W = np.zeros((8, 2 * G), dtype=np.float32)
        for n in range(8):
            for g in range(2):
                W[n, g * G:(g + 1) * G] = np.tile(W4[(n + g) % 8], rep)
        P = OQ.pack(f"w4g{G}", W)
        assert P["scales"].shape == (8, 2) and np.asarray(P["zeros"]).shape == (2, 1)
        for n in range(8):
            for g in range(2):
                src = (n + g) % 8
                assert int(np.asarray(P["scales"][n, g]).view(np.uint16)) == s4[src], (G, n, g)
                assert _decode_w4_zero(P, n, g) == z4[src], (G, n, g)
                assert [_decode_w4_codes(P, n, g * G + k) for k in range(G)] == q4[src] * rep, (G, n, g)
        assert [int(w) for w in np.asarray(P["zeros"])[:, 0]] == [num(t) for t in head["w4_zeros_words"]]
        assert int(P["qweight"][3, 0]) == num(head["w4_row3_word0"][0])
        assert int(P["qweight"][3, G // 8]) == num(head["w4_row3_group1_word0"][0])
        Wd = OQ.dequant(P)
        for n in range(8):
            for k in range(0, 2 * G, 3):
                assert Fraction(float(Wd[n, k])) == _exact_dequant(P, n, k), (G, n, k)
        W = np.zeros((3, 2 * G), dtype=np.float32)
        for n in range(3):
            for g in range(2):
                W[n, g * G:(g + 1) * G] = np.tile(W8[(n + g) % 3], rep)
        P = OQ.pack(f"w8g{G}", W)
        for n in range(3):
            for g in range(2):
                assert int(P["scales"][n, g]) == s8[(n + g) % 3], (G, n, g)
                assert [int(v) for v in P["qweight"][n, g * G:(g + 1) * G]] == q8[(n + g) % 3] * rep
        assert [int(v) for v in P["scales"][0]] == [num(t) for t in head["w8_scales_row0"]]
        assert [int(v) for v in P["scales"][2]] == [num(t) for t in head["w8_scales_row2"]]


def pin_small_groups_are_per_channel_blocks(seed=14, N=24, K=256):
    """A group of G columns is quantised as a per-channel row of its own: every block of
    G columns of a grouped pack equals the per-channel pack of that block alone (codes,
    scales and zero-points, bit for bit, each in its layout's place)."""
    W = synth.weight(seed, K, N, outliers=True)
    for G in (32, 64):
        P8, P4 = OQ.pack(f"w8g{G}", W), OQ.pack(f"w4g{G}", W)
        for b in range(K // G):
            blk = np.ascontiguousarray(W[:, b * G:(b + 1) * G])
            C8, C4 = OQ.pack("w8pc", blk), OQ.pack("w4pc", blk)
            assert np.array_equal(P8["qweight"][:, b * G:(b + 1) * G], C8["qweight"]), (G, b)
            assert np.array_equal(P8["scales"][:, b], C8["scales"]), (G, b)
            assert np.array_equal(P4["qweight"][:, b * G // 8:(b + 1) * G // 8], C4["qweight"]), (G, b)
            assert np.array_equal(np.asarray(P4["scales"]).view(np.uint16)[:, b],
                                  np.asarray(C4["scales"]).view(np.uint16)), (G, b)
            assert np.array_equal(np.asarray(P4["zeros"])[b], np.asarray(C4["zeros"]).reshape(-1)), (G, b)
        assert OQ.packed_sizes(f"w4g{G}", K, N) == (P4["qweight"].nbytes, P4["scales"].nbytes, P4["zeros"].nbytes)
        assert OQ.packed_sizes(f"w8g{G}", K, N)[:2] == (P8["qweight"].nbytes, P8["scales"].nbytes)


def pin_nibble_layout():
    head, _ = read_fixture("nibble_layout.txt")
    K, N = 16, 8
    q = np.zeros((N, K), dtype=np.uint8)
    q[0, :8] = [int(t) for t in head["codes0"]]
    q[0, 8:] = [int(t) for t in head["codes1"]]
    words = OQ._pack_nibbles_rows(q)
    assert int(words[0, 0]) == num(head["word0"][0]) and int(words[0, 1]) == num(head["word1"][0])
    z = np.zeros((N, 1), dtype=np.uint8)
    z[:, 0] = [int(t) for t in head["zeros_col"]]
    zw = OQ._pack_nibbles_rows(np.ascontiguousarray(z.T))
    assert zw.shape == (1, 1) and int(zw[0, 0]) == num(head["zeros_word"][0])
    # the same through pack(): a weight whose group-0 codes come out as 0..7 for n = 0..7
    # (w = (c - 7)/64 with lo = -7/64, hi = 8/64 in every row) and zero-point 7
    W = np.zeros((8, 128), dtype=np.float32)
    W[:, 0], W[:, 1] = -7 / 64, 8 / 64
    for n in range(8):
        W[n, 2] = (n - 7) / 64
    P = OQ.pack("w4g128", W)
    assert [_decode_w4_codes(P, n, 2) for n in range(8)] == list(range(8))
    assert int(P["zeros"][0, 0]) == 0x77777777
    assert OQ.packed_sizes("w4g128", 128, 8) == (P["qweight"].nbytes, P["scales"].nbytes, P["zeros"].nbytes)


def pin_w8_roundtrip_bound(seed=7, N=64, K=1024, G=None):
    """P1: |w - q*s| <= s/2 (+ the fp32 division slack) with the stored scale;
    the clamp never bites because 127*(1 + 2^-8) < 127.5."""
    W = synth.weight(seed, K, N)
    q, sb = OQ.quantize_w8(W, G)
    s = OQ.bf16_bits_to_f32(sb).astype(np.float64)
    g = K if G is None else G
    sfull = np.repeat(s.reshape(N, -1), g, axis=1)
    err = np.abs(W.astype(np.float64) - q.astype(np.float64) * sfull)
    bound = sfull / 2 + np.abs(W) * 2.0 ** -23
    assert np.all(err <= bound), float((err / sfull).max())
    assert int(np.abs(q.astype(int)).max()) <= 127
    # the scale is the bf16 rounding of max|w| / 127 (checked exactly)
    a = np.max(np.abs(W.reshape(N, -1, g)), axis=2)
    for n in range(0, N, 9):
        exact = _f32_fraction(a.reshape(N, -1)[n, 0]) / 127
        got = _bf16_bits_value(int(sb.reshape(N, -1)[n, 0]))
        assert abs(got - exact) <= exact * Fraction(1, 2 ** 8) * Fraction(1001, 1000)


def pin_w4_roundtrip_bound(seed=8, N=64, K=1024, G=128):
    """P2: unclamped codes are within s/2 (+ slack); clamped ones within
    s/2 + (hi - lo) * 2^-11 (the fp16 rounding of the scale)."""
    W = synth.weight(seed, K, N, outliers=True)
    q, s16, z = OQ.quantize_w4g128(W) if G == 128 else OQ.quantize_w4(W, G)
    s = np.repeat(s16.astype(np.float64), G, axis=1)
    zf = np.repeat(z.astype(np.float64), G, axis=1)
    wd = (q.astype(np.float64) - zf) * s
    err = np.abs(W.astype(np.float64) - wd)
    Wg = W.reshape(N, -1, G).astype(np.float64)
    rng_ = np.repeat(Wg.max(axis=2) - Wg.min(axis=2), G, axis=1)
    assert np.all(err <= s / 2 + rng_ * 2.0 ** -11 + np.abs(W) * 2.0 ** -22)
    assert q.max() <= 15 and z.max() <= 15


def pin_nearest_code_bruteforce():
    """P3: every unclamped code minimises |w - (c - z) * s| over all codes c."""
    rng = np.random.default_rng(99)
    for trial in range(20):
        W = (rng.standard_normal((2, 128)) * 0.02).astype(np.float32)
        q, sb = OQ.quantize_w8(W, 128)
        s = OQ.bf16_bits_to_f32(sb).astype(np.float64)
        for n in range(2):
            for k in range(0, 128, 5):
                w = float(W[n, k])
                errs = [abs(w - c * s[n, 0]) for c in range(-127, 128)]
                best = min(errs)
                assert abs(errs[int(q[n, k]) + 127] - best) <= 1e-12 * max(1.0, abs(w)), (trial, n, k)
        q4, s16, z = OQ.quantize_w4g128(W)
        for n in range(2):
            sv = float(s16[n, 0])
            span = float(W[n].max()) - float(W[n].min())
            for k in range(0, 128, 3):
                w = float(W[n, k])
                errs = [abs(w - (c - int(z[n, 0])) * sv) for c in range(16)]
                c0 = int(q4[n, k])
                if 0 < c0 < 15:
                    assert abs(errs[c0] - min(errs)) <= 1e-12, (trial, n, k)
                else:
                    assert errs[c0] <= sv / 2 + span * 2.0 ** -11 + 1e-12, (trial, n, k)


def pin_all_zero():
    """P4: an all-zero row or group stores scale 0, codes equal to the zero-point,
    and dequantises to exactly 0."""
    W = synth.weight(3, 256, 16)
    W[3, :] = 0
    W[5, 128:] = 0
    for fmt in ("w8pc", "w8g128", "w4g128"):
        P = OQ.pack(fmt, W)
        Wd = OQ.dequant(P)
        assert not np.any(Wd[3]), fmt
        sb = P["scales"].view(np.uint16)
        if fmt == "w8pc":
            assert sb[3] == 0 and not np.any(P["qweight"][3])
        else:
            assert not np.any(sb[3]) and sb[5, 1] == 0 and sb[5, 0] != 0
            assert not np.any(Wd[5, 128:])
        if fmt == "w4g128":
            for g in range(2):
                assert _decode_w4_zero(P, 3, g) == 0
            assert all(_decode_w4_codes(P, 3, k) == _decode_w4_zero(P, 3, k // 128) for k in range(256))


# ------------------------------------------------------------------- the linear
def pin_one_hot_golden():
    """P5 on the hand-derived W4 example: x = e_k selects (q - z) * s exactly."""
    W, exp_q, exp_s, exp_z = _golden_w4_weight()
    P = OQ.pack("w4g128", W)
    ks = [0, 1, 4, 5, 127, 128, 129, 130, 131, 255]
    x = synth.one_hot_activation(W.shape[1], ks)
    y = OL.ref_linear(x, P)
    for m, k in enumerate(ks):
        g = k // 128
        s = _fp16_value(np.array(exp_s[g], dtype=np.uint16).view(np.float16))
        want = (exp_q[0, k] - exp_z[g]) * s
        assert Fraction(float(y[m, 0])) == want, (k, y[m, 0], float(want))
        assert not np.any(y[m, 1:])


def pin_one_hot_random(fmt="w8g128", K=512, N=40):
    W = synth.weight(11, K, N, outliers=fmt.startswith("w4"))
    P = OQ.pack(fmt, W)
    ks = [0, 31, 32, 63, 64, 127, 128, 300, K - 1]   # both sides of every group edge size
    y = OL.ref_linear(synth.one_hot_activation(K, ks), P)
    for m, k in enumerate(ks):
        for n in range(N):
            assert Fraction(float(y[m, n])) == _exact_dequant(P, n, k), (fmt, m, n)


def pin_identity(fmt="w4g128", K=256, N=24):
    """P6: x = I gives y = dequant(W)^T exactly."""
    W = synth.weight(12, K, N, outliers=True)
    P = OQ.pack(fmt, W)
    y = OL.ref_linear(synth.identity_activation(K), P)
    for n in range(N):
        for k in range(0, K, 17):
            assert Fraction(float(y[k, n])) == _exact_dequant(P, n, k)


def pin_bruteforce(fmt, K, N=11, M=3, seed=5):
    """P7: a triple loop over exact rationals (codes decoded by hand, bf16 x decoded
    by hand) agrees with the NumPy path to fp64 rounding; N is not a multiple of
    the chunk so a dropped tail shows."""
    W = synth.weight(seed, K, N if not fmt.startswith("w4") else 16, outliers=fmt.startswith("w4"))
    N = W.shape[0]
    P = OQ.pack(fmt, W)
    x = synth.activation(seed, K, M)
    y = OL.ref_linear(x, P, chunk=5)
    for m in range(M):
        xv = [_bf16_bits_value(int(b)) for b in x[m]]
        for n in range(N):
            exact = sum(xv[k] * _exact_dequant(P, n, k) for k in range(K))
            err = abs(Fraction(float(y[m, n])) - exact)
            scale = sum(abs(xv[k] * _exact_dequant(P, n, k)) for k in range(K))
            assert err <= scale * Fraction(K + 2, 2 ** 53), (fmt, m, n, float(err))


def pin_library_factorisation(seed=21):
    """P8: per channel y = (x @ q^T) * s; group-128 y = sum_g s_g (x_g @ (q-z)_g^T),
    with plain NumPy fp64 on the codes."""
    K, N, M = 512, 48, 4
    x = synth.activation(seed, K, M)
    xf = OQ.bf16_bits_to_f32(x).astype(np.float64)
    W = synth.weight(seed, K, N)
    P = OQ.pack("w8pc", W)
    want = (xf @ P["qweight"].astype(np.float64).T) * OQ.bf16_bits_to_f32(P["scales"]).astype(np.float64)[None, :]
    assert np.allclose(OL.ref_linear(x, P), want, rtol=1e-12, atol=1e-12)
    Wo = synth.weight(seed, K, N, outliers=True)
    P4 = OQ.pack("w4g128", Wo)
    q, s16, z = OQ.unpack_w4g128(P4)
    want = np.zeros((M, N))
    for g in range(K // 128):
        d = q[:, 128 * g:128 * (g + 1)].astype(np.float64) - z[:, g:g + 1].astype(np.float64)
        want += (xf[:, 128 * g:128 * (g + 1)] @ d.T) * s16[:, g].astype(np.float64)[None, :]
    assert np.allclose(OL.ref_linear(x, P4), want, rtol=1e-12, atol=1e-12)
    P8 = OQ.pack("w8g128", W)
    sg = OQ.bf16_bits_to_f32(P8["scales"]).astype(np.float64)
    want = np.zeros((M, N))
    for g in range(K // 128):
        want += (xf[:, 128 * g:128 * (g + 1)] @ P8["qweight"][:, 128 * g:128 * (g + 1)].astype(np.float64).T) * sg[:, g][None, :]
    assert np.allclose(OL.ref_linear(x, P8), want, rtol=1e-12, atol=1e-12)


def pin_invariants():
    """P9: x = 0 gives y = 0; x * 2^j gives y * 2^j exactly; sampled columns
    equal the full product; chunking does not change the result."""
    K, N = 384, 40
    W = synth.weight(31, K, N, outliers=True)
    P = OQ.pack("w4g128", W)
    assert not np.any(OL.ref_linear(np.zeros((2, K), dtype=np.uint16), P))
    x = synth.activation(31, K, 3)
    y = OL.ref_linear(x, P)
    x4 = OQ.bf16_rne_bits(OQ.bf16_bits_to_f32(x) * np.float32(4.0))
    assert np.array_equal(OL.ref_linear(x4, P), 4.0 * y)
    cols = [0, 7, 13, 39]
    assert np.array_equal(OL.ref_linear_columns(x, P, cols), y[:, cols])
    assert np.array_equal(OL.ref_linear(x, P, chunk=7), y)


def pin_compare():
    """The tolerance rule |y - y_ref| <= 1e-2 * max(1, |y_ref|) on crafted values."""
    ref = np.array([[0.0, 0.5, 100.0, -3.0]])
    ok = OQ.bf16_rne_bits(np.array([[0.0078125, 0.5, 100.5, -3.0]], dtype=np.float32))
    st = OL.compare(ok, ref)
    assert st["fails"] == 0 and abs(st["max_ratio"] - 0.78125) < 1e-12, st
    bad = OQ.bf16_rne_bits(np.array([[0.015625, 0.5, 102.0, -3.0]], dtype=np.float32))
    st = OL.compare(bad, ref)
    assert st["fails"] == 2, st


def pin_compare_rel_rms():
    """The relative RMS ||y - y_ref||_2 / ||y_ref||_2 (the statistic of the Marlin
    benchmark page's "Fixed-input projection check") on crafted values: y = (3, 4)
    against y_ref = (6, 8) is half of a 3-4-5 triangle, so the ratio is 5 / 10 = 1/2
    exactly, each error is 50 tolerances and both elements fail.  A zero reference
    gives 0 for a zero result and +inf for any other (a relative error over a zero
    denominator)."""
    y = OQ.bf16_rne_bits(np.array([[3.0, 4.0]], dtype=np.float32))
    st = OL.compare(y, np.array([[6.0, 8.0]]))
    assert st["rel_rms"] == 0.5 and st["max_ratio"] == 50.0 and st["fails"] == 2, st
    # a single element: |y - y_ref| / |y_ref| exactly
    st = OL.compare(OQ.bf16_rne_bits(np.array([[1.5]], dtype=np.float32)), np.array([[-0.5]]))
    assert st["rel_rms"] == 4.0, st
    zero = np.zeros((2, 3))
    assert OL.compare(OQ.bf16_rne_bits(zero.astype(np.float32)), zero)["rel_rms"] == 0.0
    nz = OQ.bf16_rne_bits(np.array([[0.0, 0.25, 0.0], [0.0, 0.0, 0.0]], dtype=np.float32))
    assert OL.compare(nz, zero)["rel_rms"] == float("inf")


def pin_dispatch():
    """Token count numel/shape[-1]; fewer than 8 tokens -> GEMV."""
    assert OL.token_count((7, 5120)) == 7 and OL.token_count((2, 3, 64)) == 6
    assert OL.use_gemv(1) and OL.use_gemv(7) and not OL.use_gemv(8) and not OL.use_gemv(2048)


# ------------------------------------------------------------------- top-k, sampling
def _bf16_num(b: int):
    """A bf16 bit pattern as a Fraction, or None for NaN (an independent decoder)."""
    e, m = (b >> 7) & 0xFF, b & 0x7F
    if e == 0xFF:
        return None if m else (Fraction(10) ** 40 if not b & 0x8000 else -Fraction(10) ** 40)
    v = Fraction(m, 128) * Fraction(2) ** -126 if e == 0 else (1 + Fraction(m, 128)) * Fraction(2) ** (e - 127)
    return -v if b & 0x8000 else v


def pin_topk_golden():
    """Hand-derived example (tests/golden/topk_worked.txt): order with ties, signed
    zeros and a NaN; tokens drawn at temperatures 1, 0.5 and 0."""
    head, blocks = read_fixture("topk_worked.txt")
    bits = np.array([num(t) for t in blocks["logits"][0]], dtype=np.uint16)
    for key in ("top5", "top8"):
        want = [int(t) for t in head[key]]
        idx, kb = OT.topk_row(bits, len(want))
        assert idx.tolist() == want, (key, idx.tolist())
        assert np.array_equal(kb, bits[want])
    for k, T, u, tok in blocks["draws"]:
        idx, kb = OT.topk_row(bits, int(k))
        assert OT.sample_row(kb, idx, float(T), float(u)) == int(tok), (k, T, u, tok)


def pin_topk_rows():
    """Several rows in one call (tests/golden/topk_rows_worked.txt): each row keeps
    its own k best and draws with its own u -- row 1 is row 0 reversed and row 2 row
    0 rotated, so a draw that reused one row's u or one row's kept set for another
    lands on a different token."""
    head, blocks = read_fixture("topk_rows_worked.txt")
    L = np.array([[num(t) for t in row] for row in blocks["logits"]], dtype=np.uint16)
    k, T = int(head["k"][0]), float(head["T"][0])
    u = np.array([float(t) for t in head["u"]])
    idx, bits, tok = OT.ref_topk_sample(L, k, T, u)
    want_idx = np.array([[int(t) for t in row] for row in blocks["kept"]])
    assert np.array_equal(idx, want_idx), idx
    assert np.array_equal(bits, np.take_along_axis(L, want_idx, axis=1))
    assert tok.tolist() == [int(t) for t in head["tokens"]], tok


def pin_topk_defining_property(seed=31, V=48):
    """Brute force over pairs on a row with many ties (a small value set, both zeros,
    a NaN, infinities): for every k the kept entries beat every dropped one, and each
    kept entry beats the next, where a beats b iff a is a number and b is NaN, or
    value(a) > value(b), or the values are equal and index(a) < index(b)."""
    rng = np.random.default_rng(seed)
    pool = [0x3F80, 0xBF80, 0x4000, 0x0000, 0x8000, 0x7FC0, 0x7F80, 0xFF80, 0x3F81]
    bits = np.array([pool[i] for i in rng.integers(0, len(pool), V)], dtype=np.uint16)

    def beats(a, b):
        va, vb = _bf16_num(int(bits[a])), _bf16_num(int(bits[b]))
        if va is None or vb is None:
            return va is not None and vb is None or (va is None and vb is None and a < b)
        return va > vb or (va == vb and a < b)

    for k in range(1, V + 1):
        idx, _ = OT.topk_row(bits, k)
        kept = [int(i) for i in idx]
        assert len(set(kept)) == k
        dropped = set(range(V)) - set(kept)
        assert all(beats(a, b) for a in kept for b in dropped), k
        assert all(beats(kept[i], kept[i + 1]) for i in range(k - 1)), k


def pin_topk_sampling_closed_forms():
    """Equal logits give p = 1/k each, so u = j/k (exact) draws the (j+1)-th kept
    token (the running sum must exceed u) and u = (j + 0.5)/k the (j+1)-th as well;
    two logits d apart draw the first below 1/(1 + exp(-d/T)) and the second above;
    T = 0 and k = 1 take the best token."""
    bits = np.full(10, 0x4120, dtype=np.uint16)              # ten equal logits (10.0)
    for k in (1, 2, 4, 8):
        idx, kb = OT.topk_row(bits, k)
        assert idx.tolist() == list(range(k))
        for j in range(k):
            # the running sum after i terms is i/k (exact for these k): the first to exceed
            # j/k or (j + 1/2)/k is i = j + 1, the (j+1)-th kept token, index j
            for u in (Fraction(j, k), Fraction(2 * j + 1, 2 * k)):
                assert OT.sample_row(kb, idx, 1.0, float(u)) == j, (k, j, u)
    row = np.array([0x4000, 0x4040, 0xC000], dtype=np.uint16)   # 2, 3, -2
    idx, kb = OT.topk_row(row, 2)
    assert idx.tolist() == [1, 0]
    for T in (0.5, 1.0, 3.0):
        p1 = 1.0 / (1.0 + math.exp(-1.0 / T))
        assert OT.sample_row(kb, idx, T, p1 - 1e-9) == 1
        assert OT.sample_row(kb, idx, T, min(p1 + 1e-9, 0.999999)) == 0
        assert OT.sample_row(kb, idx, 0.0, 0.999) == 1
    one, onek = OT.topk_row(row, 1)
    assert OT.sample_row(onek, one, 1.0, 0.999) == 1
    # a non-finite best logit draws it; a NaN behind a finite best weighs nothing;
    # -inf weighs exp(-inf) = 0
    for best in (0x7F80, 0xFF80, 0x7FC0):
        assert OT.sample_row(np.array([best, 0x3F80], np.uint16), [5, 6], 1.0, 0.999) == 5
    assert OT.sample_row(np.array([0x3F80, 0x7FC0], np.uint16), [5, 6], 1.0, 0.999) == 5
    assert OT.sample_row(np.array([0x3F80, 0xFF80, 0x3F80], np.uint16), [5, 6, 7], 1.0, 0.6) == 7


# ------------------------------------------------- full-K activation permutation
def pin_activation_permutation(seed=41, K=256, N=24, M=3):
    """The gather x'[m, j] = x[m, perm[j]] against facts other than its own code:
    (a) per-channel W8 codes do not depend on the column order (one scale per row),
    so storing W[:, perm] and gathering x by the same perm reproduces the plain
    layer to fp64 rounding -- a perm that is not its own inverse catches a gather in
    the wrong direction; (b) a brute-force sum over exact rationals (codes and bf16
    decoded by hand) of x[perm[j]] * W'[n, j], with one index out of range (+0) and
    one repeated, on group-128 W4."""
    rng = np.random.default_rng(seed)
    perm = rng.permutation(K)
    assert np.any(perm[perm] != np.arange(K))            # not an involution
    W = synth.weight(seed, K, N)
    x = synth.activation(seed, K, M)
    y0 = OL.ref_linear(x, OQ.pack("w8pc", W))
    y1 = OL.ref_linear_perm(x, OQ.pack("w8pc", np.ascontiguousarray(W[:, perm])), perm)
    assert np.allclose(y1, y0, rtol=1e-12, atol=1e-12)
    # (b) tiny brute force with an out-of-range and a repeated index
    K2, N2 = 128, 8
    W2 = synth.weight(seed + 1, K2, N2, outliers=True)
    P2 = OQ.pack("w4g128", W2)
    x2 = synth.activation(seed + 1, K2, 2)
    p2 = rng.permutation(K2)
    p2[5] = K2 + 3                                       # reads +0
    p2[9] = p2[10]                                       # a plain gather repeats
    y2 = OL.ref_linear_perm(x2, P2, p2)
    for m in range(2):
        xv = [_bf16_bits_value(int(b)) for b in x2[m]]
        for n in range(N2):
            terms = [(xv[int(p2[j])] if 0 <= p2[j] < K2 else Fraction(0)) * _exact_dequant(P2, n, j)
                     for j in range(K2)]
            exact = sum(terms)
            bound = sum(abs(t) for t in terms) * Fraction(K2 + 2, 2 ** 53)
            assert abs(Fraction(float(y2[m, n])) - exact) <= bound, (m, n)


# ------------------------------------------------------ grouped layer, SiLU gate
def pin_silu_closed_forms():
    """silu(v) = v sigmoid(v): sigmoid(ln 3) = 3/4 exactly, so silu(+-ln 3) = (3/4) ln 3
    and -(1/4) ln 3; silu(0) = 0; silu(v) - silu(-v) = v (sigmoid(v) + sigmoid(-v) = 1);
    far tails: silu(50) = 50 in fp64 and silu(-800) = -0.0 (exp overflows, no NaN); the
    gated product silu(g) * u of [g | u] at g = ln 3, u = 4 is 3 ln 3."""
    l3 = math.log(3.0)
    v = OM.silu(np.array([0.0, l3, -l3, 50.0, -800.0]))
    assert v[0] == 0.0
    assert abs(v[1] - 0.75 * l3) <= 4e-16 * l3 and abs(v[2] + 0.25 * l3) <= 4e-16 * l3, v
    assert v[3] == 50.0 and v[4] == 0.0 and math.copysign(1.0, v[4]) < 0
    xs = np.linspace(-12.0, 12.0, 97)
    assert np.allclose(OM.silu(xs) - OM.silu(-xs), xs, rtol=1e-14, atol=1e-14)
    h = OM.silu_mul(np.array([[l3, -l3, 4.0, 2.0]]))
    assert abs(h[0, 0] - 3.0 * l3) <= 1e-15 * 3 * l3 and abs(h[0, 1] + 0.5 * l3) <= 1e-15, h


def pin_moe_grouping(seed=51, K=256, N=24):
    """Each row meets its own expert's weight: experts with distinct weights, one-hot
    rows x[t] = e_{k_t}, so y[t, n] must be expert e(t)'s exactly dequantised weight at
    (n, k_t) (decoded by hand from the packed bytes, independently of the oracle's
    dequantiser); an empty expert between two others; one expert over all rows is the
    dense layer; offsets that do not rise from 0 to T are refused."""
    E, T = 4, 9
    off = np.array([0, 3, 3, 7, 9])                       # expert 1 has no rows
    for fmt in ("w8pc", "w4g128"):
        Ps = [OQ.pack(fmt, synth.weight(seed + e, K, N, fmt == "w4g128")) for e in range(E)]
        ks = [(7 * t + 3) % K for t in range(T)]
        x = synth.one_hot_activation(K, ks)
        y = OM.ref_moe_linear(x, off, Ps)
        for t in range(T):
            e = int(np.searchsorted(off, t, side="right")) - 1
            for n in range(N):
                assert Fraction(float(y[t, n])) == _exact_dequant(Ps[e], n, ks[t]), (fmt, t, n)
        xr = synth.activation(seed, K, T)
        assert np.array_equal(OM.ref_moe_linear(xr, [0, T], Ps[:1]), OL.ref_linear(xr, Ps[0]))
    for bad in ([1, 3, 9], [0, 5, 3, 9], [0, 3, 8]):
        try:
            OM.check_offsets(bad, T)
        except ValueError:
            continue
        raise AssertionError(f"offsets {bad} accepted")


def pin_f16_activations(seed=61):
    """FP16 activations: the fp16 decode against the pins' own hand-written decoder on
    every finite bit pattern and on hand values; the layer on fp16 x -- one-hot rows
    give the exact dequantised weight, random rows agree with a rational triple loop --
    and the parity statistic reading fp16 results."""
    b = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16)
    finite = ((b >> 10) & 0x1F) != 0x1F
    dec = OL.f16_bits_to_f64(b[finite])
    for i in range(0, int(finite.sum()), 97):
        assert Fraction(float(dec[i])) == _fp16_value(np.array(b[finite][i], dtype=np.uint16).view(np.float16)), hex(b[finite][i])
    hand = OL.f16_bits_to_f64(np.array([0x3C00, 0xC000, 0x7BFF, 0x0400, 0x0001, 0x3555], dtype=np.uint16))
    assert [Fraction(float(v)) for v in hand] == [1, -2, 65504, Fraction(1, 2 ** 14), Fraction(1, 2 ** 24),
                                                 Fraction(1365, 4096)]
    for fmt, K in (("w4g128", 256), ("w8pc", 96), ("w8g32", 64)):
        W = synth.weight(seed, K, 16, outliers=fmt.startswith("w4"))
        P = OQ.pack(fmt, W)
        ks = [0, 31, 32, K - 1]
        x = np.zeros((len(ks), K), dtype=np.uint16)
        for m, k in enumerate(ks):
            x[m, k] = 0x3C00                                  # fp16 1.0
        y = OL.ref_linear(x, P, act="f16")
        for m, k in enumerate(ks):
            for n in range(16):
                assert Fraction(float(y[m, n])) == _exact_dequant(P, n, k), (fmt, k, n)
        x = synth.activation_f16(seed, K, 3)
        y = OL.ref_linear(x, P, chunk=5, act="f16")
        for m in range(3):
            xv = [_fp16_value(np.array(v, dtype=np.uint16).view(np.float16)) for v in x[m]]
            for n in range(0, 16, 3):
                exact = sum(xv[k] * _exact_dequant(P, n, k) for k in range(K))
                scale = sum(abs(xv[k] * _exact_dequant(P, n, k)) for k in range(K))
                assert abs(Fraction(float(y[m, n])) - exact) <= scale * Fraction(K + 2, 2 ** 53), (fmt, m, n)
    st = OL.compare(np.array([0x3C01, 0x5640, 0x0000], dtype=np.uint16), np.array([1.0, 100.0, 0.0]), act="f16")
    assert st["fails"] == 0 and abs(st["max_ratio"] - 2.0 ** -10 / 1e-2) < 1e-12, st
    st = OL.compare(np.array([0x3C00], dtype=np.uint16), np.array([1.5]), act="f16")
    assert st["fails"] == 1 and abs(st["max_ratio"] - 0.5 / 0.015) < 1e-9, st


def pin_residual(seed=62):
    """The residual epilogue: r = 0 leaves the layer, x = 0 gives r exactly, and a one-hot
    row gives the dequantised weight plus r (both exact rationals); in fp16 as in bf16."""
    for fmt, K in (("w8pc", 96), ("w4g128", 128)):
        W = synth.weight(seed, K, 16, outliers=fmt.startswith("w4"))
        P = OQ.pack(fmt, W)
        x = synth.activation(seed, K, 3)
        zero = np.zeros((3, 16), dtype=np.uint16)
        assert np.array_equal(OL.ref_linear_residual(x, P, zero), OL.ref_linear(x, P))
        r = synth.activation(seed + 1, 16, 3)
        y = OL.ref_linear_residual(np.zeros((3, K), dtype=np.uint16), P, r)
        for m in range(3):
            for n in range(16):
                assert Fraction(float(y[m, n])) == _bf16_bits_value(int(r[m, n])), (fmt, m, n)
        ks = [0, 5, K - 1]
        y = OL.ref_linear_residual(synth.one_hot_activation(K, ks), P, r)
        for m, k in enumerate(ks):
            for n in range(16):
                want = _exact_dequant(P, n, k) + _bf16_bits_value(int(r[m, n]))
                assert Fraction(float(y[m, n])) == want, (fmt, k, n)
        r16 = synth.activation_f16(seed + 1, 16, 3)
        x16 = np.zeros((3, K), dtype=np.uint16)
        y = OL.ref_linear_residual(x16, P, r16, act="f16")
        for m in range(3):
            for n in range(16):
                assert Fraction(float(y[m, n])) == _fp16_value(np.array(r16[m, n], dtype=np.uint16).view(np.float16))


ALL_PINS = [
    pin_bf16_rounding, pin_golden_w8pc, pin_golden_w4g128, pin_nibble_layout,
    pin_w8_roundtrip_bound, lambda: pin_w8_roundtrip_bound(G=128), pin_w4_roundtrip_bound,
    pin_nearest_code_bruteforce, pin_all_zero, pin_one_hot_golden,
    lambda: pin_one_hot_random("w8pc"), lambda: pin_one_hot_random("w8g128"),
    lambda: pin_one_hot_random("w4g128"), pin_identity,
    lambda: pin_bruteforce("w8pc", 48), lambda: pin_bruteforce("w8g128", 128),
    lambda: pin_bruteforce("w4g128", 128), pin_library_factorisation, pin_invariants,
    pin_compare, pin_compare_rel_rms, pin_dispatch, pin_topk_golden, pin_topk_rows,
    pin_topk_defining_property,
    pin_topk_sampling_closed_forms, pin_activation_permutation, pin_silu_closed_forms, pin_moe_grouping,
    pin_golden_w4pc, pin_w4pc_one_group_is_group128, pin_w4pc_roundtrip_bound,
    lambda: pin_bruteforce("w4pc", 64), lambda: pin_one_hot_random("w4pc"),
    pin_golden_small_groups, pin_small_groups_are_per_channel_blocks,
    lambda: pin_w8_roundtrip_bound(G=32), lambda: pin_w4_roundtrip_bound(G=32),
    lambda: pin_w4_roundtrip_bound(G=64),
    lambda: pin_bruteforce("w8g32", 64), lambda: pin_bruteforce("w8g64", 128),
    lambda: pin_bruteforce("w4g32", 96), lambda: pin_bruteforce("w4g64", 128),
    lambda: pin_one_hot_random("w8g32"), lambda: pin_one_hot_random("w8g64"),
    lambda: pin_one_hot_random("w4g32"), lambda: pin_one_hot_random("w4g64"),
    pin_f16_activations, pin_residual,
]


def run_all_pins():
    for p in ALL_PINS:
        p()
