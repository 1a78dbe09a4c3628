"""The C-ABI library loads, exports every symbol include/wq.h declares, and its
host-only logic (sizes, dispatch rule, tuner choice, tuner cache, argument
validation) behaves as documented.  No device work: CPU only."""
import ctypes as C
import os
import re

import pytest

import oracle.quant as OQ

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "wq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(wq_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported(wqlib):
    names = _declared()
    assert len(names) >= 19, names
    for n in names:
        assert hasattr(wqlib.lib, n), n


def test_abi_version_and_status_strings(wqlib):
    assert wqlib.wq_abi_version() == 1
    for st in range(8):
        assert wqlib.wq_status_string(st)
    assert wqlib.wq_status_string(99) == "unknown status"


@pytest.mark.parametrize("fmt", OQ.FORMATS)
@pytest.mark.parametrize("K,N", [(1024, 1024), (5120, 27648), (13824, 5120), (5120, 151936), (384, 40)])
def test_packed_sizes_match_the_oracle_layout(wqlib, fmt, K, N):
    if fmt == "w4g128" and N % 8:
        pytest.skip("W4 needs N % 8 == 0")
    assert wqlib.wq_packed_sizes(fmt, wqlib.CANONICAL, K, N) == OQ.packed_sizes(fmt, K, N)
    q, s, z = wqlib.wq_packed_sizes(fmt, wqlib.GFX950, K, N)
    n16, G = -(-N // 16), K // 128
    assert q == OQ.packed_sizes(fmt, K, N)[0]
    assert s == (2 * N if fmt == "w8pc" else 2 * n16 * 16 * G)
    assert z == (n16 * G * 8 if fmt == "w4g128" else 0)


@pytest.mark.parametrize("fmt,K,N,status", [
    ("w8pc", 1000, 64, 2),      # K % 16
    ("w8g128", 1040, 64, 2),    # K % 128
    ("w4g128", 1024, 60, 2),    # N % 8
    ("w8pc", 0, 64, 1),
    (8, 1024, 64, 2),           # unknown format
])
def test_packed_sizes_rejects_bad_shapes(wqlib, fmt, K, N, status):
    with pytest.raises(wqlib.WqError) as e:
        wqlib.wq_packed_sizes(fmt, wqlib.CANONICAL, K, N)
    assert e.value.status == status
    assert wqlib.wq_last_error()


def test_gemv_max_split(wqlib):
    assert wqlib.wq_gemv_max_split("w8pc", 1024) == 1
    assert wqlib.wq_gemv_max_split("w8pc", 5120) == 4       # 5 slices of 1024
    assert wqlib.wq_gemv_max_split("w8pc", 27648) == 16     # 27 slices
    assert wqlib.wq_gemv_max_split("w4g128", 5120) == 2     # 3 slices of 2048 (ragged)
    assert wqlib.wq_gemv_max_split("w8g128", 5120 * 16) == 32
    assert wqlib.wq_gemv_max_split("w8pc", 1000) == -1


def test_gemv_max_waves(wqlib):
    for fmt in ("w8pc", "w8g128", "w4g128"):
        for rows in (4, 8, 16):
            caps = [wqlib.wq_gemv_max_waves(fmt, m, rows) for m in range(1, 8)]
            assert all(c in (4, 8, 16) for c in caps) and caps == sorted(caps, reverse=True)
        assert wqlib.wq_gemv_max_waves(fmt, 1, 4) == 16
    assert wqlib.wq_gemv_max_waves("w8pc", 0, 4) == -1 and wqlib.wq_gemv_max_waves("w8pc", 8, 4) == -1
    assert wqlib.wq_gemv_max_waves(9, 1, 4) == -1 and wqlib.wq_gemv_max_waves("w8pc", 1, 5) == -1
    # the slice-prefetch flag: offered while 4 * rows + M * (8 int8 / 16 uint4 x words) <= 48
    pf = wqlib.GEMV_PREFETCH
    for fmt, xw in (("w8pc", 8), ("w8g128", 8), ("w4g128", 16)):
        for rows in (4, 8, 16):
            for m in range(1, 8):
                cap = wqlib.wq_gemv_max_waves(fmt, m, rows | pf)
                offered = 4 * rows + m * xw <= 48
                assert (cap > 0) == offered, (fmt, rows, m, cap)
                if offered:
                    assert cap <= wqlib.wq_gemv_max_waves(fmt, m, rows)
    assert wqlib.wq_gemv_max_waves("w8pc", 1, pf) == -1                     # flag without rows
    # the matrix-core GEMV: 16 NB rows with NB in 1, 2, 4, up to 8 waves
    mf = wqlib.GEMV_MFMA
    for m in range(1, 8):
        for rows in (16, 32, 64):
            for fmt in ("w8pc", "w8g128", "w4g128"):
                assert wqlib.wq_gemv_max_waves(fmt, m, rows | mf) == 8
    for rows in (0, 4, 8, 48, 128, 256):
        assert wqlib.wq_gemv_max_waves("w4g128", 1, rows | mf) == -1
    assert wqlib.wq_gemv_max_waves("w4g128", 1, 16 | mf | pf) == -1


def test_dispatch_threshold(wqlib):
    assert [wqlib.wq_dispatch_kind(m) for m in (0, 1, 7, 8, 2048)] == [-1, 0, 0, 1, 1]


def test_tuner_pick_min_with_ties_to_the_later_candidate(wqlib):
    assert wqlib.wq_tune_pick([5.0, 3.0, 4.0]) == 1
    assert wqlib.wq_tune_pick([5.0, 3.0, 3.0, 4.0]) == 2          # tie -> later (">=")
    assert wqlib.wq_tune_pick([2.0, -1.0, 2.0, -1.0]) == 2        # -1 = not run
    assert wqlib.wq_tune_pick([-1.0, -1.0]) == -1
    assert wqlib.lib.wq_tune_pick(None, 0) == -1


def test_tuner_cache_roundtrip_and_corrupt_file(wqlib, tmp_path):
    tag = "gfx950:256"
    wqlib.wq_tune_cache_clear()
    assert wqlib.wq_tune_cache_get("w8pc", 5120, 27648, 1, 0, tag) is None
    wqlib.wq_tune_cache_set("w8pc", 5120, 27648, 1, 0, wqlib.gemv_cache_value(4, 8, 16), tag)
    wqlib.wq_tune_cache_set("w4g128", 13824, 5120, 1, 0, 16, tag)
    with pytest.raises(wqlib.WqError):
        wqlib.wq_tune_cache_set("w8pc", 5120, 27648, 1, 0, wqlib.gemv_cache_value(3, 4), tag)
    with pytest.raises(wqlib.WqError):
        wqlib.wq_tune_cache_set("w8pc", 5120, 27648, 1, 0, wqlib.gemv_cache_value(4, 17), tag)
    with pytest.raises(wqlib.WqError):
        wqlib.wq_tune_cache_set("w8pc", 5120, 27648, 1, 0, wqlib.gemv_cache_value(4, 2, 6), tag)
    wqlib.wq_tune_cache_set("w8pc", 5120, 27648, 2048, 1, 2, tag)
    with pytest.raises(wqlib.WqError):
        wqlib.wq_tune_cache_set("w8pc", 5120, 27648, 1, 0, 3, tag)    # not a power of two
    with pytest.raises(wqlib.WqError):
        wqlib.wq_tune_cache_set("w8pc", 5120, 27648, 8, 1, wqlib.GEMM_TILES + 1, tag)  # no such tile
    p = str(tmp_path / "tune.txt")
    wqlib.wq_tune_cache_save(p)
    wqlib.wq_tune_cache_clear()
    assert wqlib.wq_tune_cache_get("w8pc", 5120, 27648, 1, 0, tag) is None
    wqlib.wq_tune_cache_load(p)
    assert wqlib.wq_tune_cache_get("w8pc", 5120, 27648, 1, 0, tag) == 4 | (8 << 8) | (16 << 16)
    assert wqlib.wq_tune_cache_get("w4g128", 13824, 5120, 1, 0, tag) == 16
    assert wqlib.wq_tune_cache_get("w8pc", 5120, 27648, 2048, 1, tag) == 2
    assert wqlib.wq_tune_cache_get("w8pc", 5120, 27648, 1, 0, "gfx942:304") is None
    bad = tmp_path / "bad.txt"
    bad.write_text("gfx950:256 0 5120 27648 1 0 4\nthis is not an entry\n")
    wqlib.wq_tune_cache_clear()
    with pytest.raises(wqlib.WqError) as e:
        wqlib.wq_tune_cache_load(str(bad))
    assert e.value.status == 7
    assert wqlib.wq_tune_cache_get("w8pc", 5120, 27648, 1, 0, tag) is None   # unchanged on failure
    with pytest.raises(wqlib.WqError) as e:
        wqlib.wq_tune_cache_load(str(tmp_path / "missing.txt"))
    assert e.value.status == 7


def _desc(wqlib, fmt=0, layout=1, K=1024, N=1024, q=0x1000, s=0x2000, z=0):
    return wqlib.WqWeightC(fmt, layout, K, N, q, s, z)


def test_validation_rejects_before_any_device_work(wqlib):
    """Bad arguments are refused on the host (nothing is launched, so this runs
    without a GPU)."""
    L = wqlib.lib
    d = _desc(wqlib)
    x, y = C.c_void_p(0x10000), C.c_void_p(0x20000)
    assert L.wq_gemv(None, x, 1, y, 1, None, 0, None) == 1                  # NULL weight
    assert L.wq_gemv(C.byref(d), x, 8, y, 1, None, 0, None) == 1            # M > 7
    assert L.wq_gemv(C.byref(d), x, 0, y, 1, None, 0, None) == 1            # M < 1
    assert L.wq_gemv(C.byref(d), None, 1, y, 1, None, 0, None) == 1         # NULL x
    assert L.wq_gemv(C.byref(d), C.c_void_p(0x10008), 1, y, 1, None, 0, None) == 3   # x misaligned
    assert L.wq_gemv(C.byref(d), x, 1, y, 3, None, 0, None) == 1            # split not pow2
    assert L.wq_gemv(C.byref(d), x, 1, y, 2, None, 0, None) == 1            # split > K slices (1)
    dk = _desc(wqlib, K=8192)
    assert L.wq_gemv(C.byref(dk), x, 1, y, 4, None, 0, None) == 4           # no workspace
    assert L.wq_gemv(C.byref(dk), x, 1, y, 4, C.c_void_p(0x30000), 16, None) == 4   # too small
    assert L.wq_gemv(C.byref(dk), x, 1, y, 4, C.c_void_p(0x30004), 1 << 20, None) == 3  # ws misaligned
    assert L.wq_gemv_ex(C.byref(d), x, 1, y, 1, 17, 0, None, 0, None) == 1  # waves > 16
    assert L.wq_gemv_ex(C.byref(d), x, 1, y, 1, 1, 5, None, 0, None) == 1   # rows not 4/8/16
    assert L.wq_gemv_ex(C.byref(d), x, 1, y, 0, 4, 0, None, 0, None) == 1   # split must be given
    assert L.wq_gemv_ex(C.byref(d), x, 1, y, 1, 1, 0x100, None, 0, None) == 1   # prefetch without rows
    assert L.wq_gemv_ex(C.byref(d), x, 1, y, 1, 1, 16 | 0x100, None, 0, None) == 2  # prefetch not offered
    assert L.wq_gemv_ex(C.byref(d), x, 1, y, 1, 9, 16 | 0x200, None, 0, None) == 2  # matrix-core GEMV: <= 8 waves
    assert L.wq_gemv_ex(C.byref(d), x, 1, y, 1, 1, 8 | 0x200, None, 0, None) == 1   # not 16 NB rows
    assert L.wq_gemv_ex(C.byref(d), x, 1, y, 1, 1, 16 | 0x300, None, 0, None) == 1  # both flags
    dc = _desc(wqlib, layout=0)
    assert L.wq_gemv(C.byref(dc), x, 1, y, 1, None, 0, None) == 2           # canonical layout
    dq = _desc(wqlib, q=0x1004)
    assert L.wq_gemv(C.byref(dq), x, 1, y, 1, None, 0, None) == 3           # qweight misaligned
    d4 = _desc(wqlib, fmt=2)
    assert L.wq_gemv(C.byref(d4), x, 1, y, 1, None, 0, None) == 1           # W4 without zeros
    dsa = _desc(wqlib, fmt=1, s=0x2002)
    assert L.wq_gemv(C.byref(dsa), x, 1, y, 1, None, 0, None) == 3          # tiled scales misaligned
    assert L.wq_gemm(C.byref(d), x, 16, y, wqlib.GEMM_TILES + 1, None, 0, None) == 1  # bad tile
    d8 = _desc(wqlib, fmt=1, K=64)
    assert L.wq_gemv(C.byref(d8), x, 1, y, 1, None, 0, None) == 2           # g128 with K=64
    assert L.wq_pack(None, C.byref(dc), None) == 1
    assert L.wq_pack_bf16(None, C.byref(dc), None) == 1
    assert L.wq_pack_bf16(C.c_void_p(0x10004), C.byref(dc), None) == 3       # bf16 w not 8-byte aligned
    assert L.wq_pack_bf16(C.c_void_p(0x10008), C.byref(d), None) == 2        # out not canonical
    assert L.wq_repack(C.byref(d), C.byref(d), None) == 2                   # src not canonical
    assert L.wq_repack(C.byref(dc), C.byref(_desc(wqlib, q=0x1000)), None) == 1  # in place
    n = C.c_size_t()
    assert L.wq_workspace_size(C.byref(d), 1, C.byref(n)) == 0 and n.value == 32 * 1024 * 4
    assert L.wq_workspace_size(C.byref(d), 7, C.byref(n)) == 0 and n.value == 32 * 7 * 1024 * 4
    # M >= 8: split-K partials -- the skinny GEMM (split <= 16, split * M <= 1024, M <= 128)
    # and the LDS-DMA tiles (split <= 16 for the 64-row tiles, at most 512 workgroups,
    # <= 256 MiB): 4 column tiles of 256 x 64-row tiles x 16 stays within 512 workgroups
    assert L.wq_workspace_size(C.byref(d), 8, C.byref(n)) == 0 and n.value == 16 * 8 * 1024 * 4
    assert L.wq_workspace_size(C.byref(d), 64, C.byref(n)) == 0 and n.value == 16 * 64 * 1024 * 4
    assert L.wq_workspace_size(C.byref(d), 128, C.byref(n)) == 0 and n.value == 16 * 128 * 1024 * 4
    assert L.wq_workspace_size(C.byref(d), 129, C.byref(n)) == 0 and n.value == 16 * 129 * 1024 * 4
    big = _desc(wqlib, K=5120, N=27648)
    assert L.wq_workspace_size(C.byref(big), 512, C.byref(n)) == 0 and n.value == 2 * 512 * 27648 * 4
    # 864 tiles = 3 rounds of 256 CUs + 96: tile 13 splits those 96 over K in 2 (a
    # 256 x 256 fp32 block per range; sized for 256 CUs when no device is visible)
    tail = 2 * 96 * 256 * 256 * 4
    assert L.wq_workspace_size(C.byref(big), 2048, C.byref(n)) == 0 and n.value == tail
    assert L.wq_workspace_size(C.byref(big), 1024, C.byref(n)) == 0 and n.value == 0   # 432 tiles: 176 left over
    # group-128: 128 x 256 tiles (the exact kernel's second accumulator set), and x in
    # fp16 (M x K x 2) after the partials, then the M row scales (fp32).  M = 2048: 1728 tiles, a last round of 192
    # (more than half the CUs: not split); M = 512: 432 tiles, no split either
    big4 = _desc(wqlib, fmt=2, K=5120, N=27648)
    assert L.wq_workspace_size(C.byref(big4), 2048, C.byref(n)) == 0 and n.value == 2048 * 5120 * 2 + 2048 * 4
    assert L.wq_workspace_size(C.byref(big4), 512, C.byref(n)) == 0 and n.value == 512 * 5120 * 2 + 512 * 4
    # 16 x 17 = 272 tiles of 128 x 256: 16 left over, split over K in 4 (a 128 x 256
    # fp32 block per range)
    tail4 = _desc(wqlib, fmt=2, K=5120, N=17 * 256)
    assert L.wq_workspace_size(C.byref(tail4), 2048, C.byref(n)) == 0 and \
        n.value == 4 * 16 * 128 * 256 * 4 + 2048 * 5120 * 2 + 2048 * 4


def test_lm_head_topk_validation_and_workspace(wqlib):
    """The LM head + top-k entry point refuses bad arguments on the host, and its
    workspace is the layer's, then the bf16 logits, then 8-byte candidates (k per
    2048-logit chunk), each part 256-byte aligned."""
    L = wqlib.lib
    n = C.c_size_t()
    d = _desc(wqlib, fmt=1, K=5120, N=151936)
    lin = C.c_size_t()
    assert L.wq_workspace_size(C.byref(d), 1, C.byref(lin)) == 0
    r = lambda b: (b + 255) // 256 * 256
    assert L.wq_lm_head_topk_workspace_size(C.byref(d), 1, 50, C.byref(n)) == 0
    assert n.value == r(r(lin.value) + 151936 * 2) + 75 * 50 * 8
    assert L.wq_lm_head_topk_workspace_size(C.byref(d), 1, 0, C.byref(n)) == 1       # k < 1
    assert L.wq_lm_head_topk_workspace_size(C.byref(d), 1, 65, C.byref(n)) == 1      # k > 64
    assert L.wq_lm_head_topk_workspace_size(C.byref(d), 0, 5, C.byref(n)) == 1       # M < 1
    small = _desc(wqlib, fmt=0, K=64, N=40)
    assert L.wq_lm_head_topk_workspace_size(C.byref(small), 1, 41, C.byref(n)) == 1  # k > N
    wide = _desc(wqlib, fmt=0, K=64, N=300000)
    assert L.wq_lm_head_topk_workspace_size(C.byref(wide), 1, 64, C.byref(n)) == 2   # 147 chunks x 64 > 8192
    x, u = C.c_void_p(0x10000), C.c_void_p(0x20000)
    tv, ti, tk, ws = C.c_void_p(0x30000), C.c_void_p(0x40000), C.c_void_p(0x50000), C.c_void_p(0x100000)
    big = 1 << 30
    call = lambda T, **kw: L.wq_lm_head_topk(C.byref(kw.get("d", d)), kw.get("x", x), 1, kw.get("k", 8), T,
                                             kw.get("u", u), tv, kw.get("ti", ti), tk, kw.get("ws", ws),
                                             kw.get("wsb", big), None)
    assert call(-1.0) == 1                                             # negative temperature
    assert call(float("inf")) == 1 and call(float("nan")) == 1
    assert call(1.0, u=None) == 1 and call(1.0, x=None) == 1
    assert call(1.0, ti=C.c_void_p(0x40002)) == 3                      # int32 output misaligned
    assert call(1.0, ws=C.c_void_p(0x100010)) == 3                     # workspace not 256-aligned
    assert call(1.0, wsb=1024) == 4 and call(1.0, ws=None) == 4        # workspace too small / missing
    assert call(1.0, k=0) == 1
    canon = _desc(wqlib, fmt=1, layout=0, K=5120, N=151936)
    assert call(1.0, d=canon) == 2                                     # not the gfx950 layout


def test_linear_perm_validation_and_workspace(wqlib):
    """The activation-permutation entry point refuses bad arguments on the host; its
    workspace is the layer's own, then x' bf16 [M][K] from a 256-byte boundary."""
    L = wqlib.lib
    n, lin = C.c_size_t(), C.c_size_t()
    r = lambda b: (b + 255) // 256 * 256
    for fmt, M in ((0, 1), (2, 4), (1, 2048)):
        d = _desc(wqlib, fmt=fmt, K=5120, N=27648)
        assert L.wq_workspace_size(C.byref(d), M, C.byref(lin)) == 0
        assert L.wq_linear_perm_workspace_size(C.byref(d), M, C.byref(n)) == 0
        assert n.value == r(lin.value) + M * 5120 * 2
    d = _desc(wqlib, fmt=0, K=5120, N=27648)
    assert L.wq_linear_perm_workspace_size(C.byref(d), 0, C.byref(n)) == 1          # M < 1
    x, perm, y, ws = C.c_void_p(0x10000), C.c_void_p(0x20000), C.c_void_p(0x30000), C.c_void_p(0x100000)
    big = 1 << 30
    call = lambda **kw: L.wq_linear_perm(C.byref(kw.get("d", d)), kw.get("x", x), kw.get("perm", perm),
                                         kw.get("M", 1), kw.get("y", y), kw.get("ws", ws), kw.get("wsb", big), None)
    assert call(perm=None) == 1 and call(x=None) == 1 and call(y=None) == 1
    assert call(M=0) == 1
    assert call(perm=C.c_void_p(0x20002)) == 3                          # int32 index misaligned
    assert call(x=C.c_void_p(0x10001)) == 3
    assert call(ws=C.c_void_p(0x100010)) == 3                           # workspace not 256-aligned
    assert call(wsb=1024) == 4 and call(ws=None) == 4                   # workspace too small / missing
    assert call(d=_desc(wqlib, fmt=0, layout=0, K=5120, N=27648)) == 2  # not the gfx950 layout


def test_binding_constants_match_the_header(wqlib):
    """The binding's copies of the header's array sizes and limits (a mismatch once let
    wq_tune write past the binding's latency buffer)."""
    import re
    import gemm_decode_amd.wq as wq
    hdr = open(os.path.join(ROOT, "include", "wq.h")).read()
    defs = dict(re.findall(r"#define (WQ_[A-Z_]+) (\d+)", hdr))
    assert int(defs["WQ_GEMM_TILES"]) == wq.GEMM_TILES
    assert int(defs["WQ_TUNE_LAT_SLOTS"]) == wq.TUNE_LAT_SLOTS
    assert int(re.search(r"#define WQ_GEMV_PREFETCH (0x[0-9a-fA-F]+)", hdr).group(1), 16) == wq.GEMV_PREFETCH
    assert int(re.search(r"#define WQ_GEMV_MFMA (0x[0-9a-fA-F]+)", hdr).group(1), 16) == wq.GEMV_MFMA
    assert wq.TUNE_LAT_SLOTS >= max(wq.GEMM_TILES, len(wq.SPLIT_GRID))
    assert int(defs["WQ_EPILOGUE_NONE"]) == wq.EPILOGUE_NONE and int(defs["WQ_EPILOGUE_SILU_MUL"]) == wq.EPILOGUE_SILU_MUL
    m = re.search(r"#define WQ_STATIC_SCRATCH_BYTES \((\d+)u << (\d+)\)", hdr)
    assert m and int(m.group(1)) << int(m.group(2)) == wq.STATIC_SCRATCH_BYTES



def test_moe_linear_host_validation(wqlib):
    """wq_moe_linear refuses bad arguments on the host, before any device work."""
    L = wqlib.lib
    p = C.c_void_p(1 << 20)
    d = wqlib.WqWeightC(wqlib.FMT["w4g128"], wqlib.GFX950, 1024, 96, 1 << 20, 1 << 20, 1 << 20)
    assert L.wq_moe_linear(C.byref(d), 0, p, p, 8, p, 0, None) == 1                 # E = 0
    assert L.wq_moe_linear(C.byref(d), 4, p, p, -1, p, 0, None) == 1                # T < 0
    assert L.wq_moe_linear(C.byref(d), 4, p, p, 8, p, 7, None) == 1                 # unknown epilogue
    assert L.wq_moe_linear(C.byref(d), 4, None, p, 8, p, 0, None) == 1              # NULL x
    assert L.wq_moe_linear(C.byref(d), 4, C.c_void_p((1 << 20) + 8), p, 8, p, 0, None) == 3   # x misaligned
    d80 = wqlib.WqWeightC(wqlib.FMT["w4g128"], wqlib.GFX950, 1024, 80, 1 << 20, 1 << 20, 1 << 20)
    assert L.wq_moe_linear(C.byref(d80), 4, p, p, 8, p, 1, None) == 2               # gated: N % 32
    d2 = wqlib.WqWeightC(wqlib.FMT["w8pc"], wqlib.GFX950, 1040, 64, 1 << 20, 1 << 20, 0)
    assert L.wq_moe_linear(C.byref(d2), 4, p, p, 8, p, 0, None) == 2                # K % 128
    d3 = wqlib.WqWeightC(wqlib.FMT["w8pc"], wqlib.CANONICAL, 1024, 64, 1 << 20, 1 << 20, 0)
    assert L.wq_moe_linear(C.byref(d3), 4, p, p, 8, p, 0, None) == 2                # layout
    assert L.wq_moe_linear(C.byref(d2), 4, p, p, 0, p, 0, None) != 0                # (K % 128 first)


def test_w4_per_channel_host_side(wqlib):
    """INT4 per channel (fmt 3): canonical sizes as the oracle's, the gfx950 layout the
    size of group-128's (each row's scale and zero-point repeated per group), the shape
    rules (K % 128, N % 8), zeros required, and the tuner cache shared with group-128 W4
    (the same kernels run both)."""
    for K, N in ((1024, 1024), (5120, 27648), (13824, 5120)):
        assert wqlib.wq_packed_sizes("w4pc", wqlib.CANONICAL, K, N) == OQ.packed_sizes("w4pc", K, N)
        assert wqlib.wq_packed_sizes("w4pc", wqlib.GFX950, K, N) == wqlib.wq_packed_sizes("w4g128", wqlib.GFX950, K, N)
    for K, N in ((1040, 64), (1024, 60)):
        with pytest.raises(wqlib.WqError) as e:
            wqlib.wq_packed_sizes("w4pc", wqlib.CANONICAL, K, N)
        assert e.value.status == 2
    L = wqlib.lib
    x, y = C.c_void_p(0x10000), C.c_void_p(0x20000)
    d = wqlib.WqWeightC(wqlib.FMT["w4pc"], wqlib.GFX950, 1024, 64, 0x1000, 0x2000, 0)
    assert L.wq_gemv(C.byref(d), x, 1, y, 1, None, 0, None) == 1          # W4 without zeros
    assert wqlib.wq_gemv_max_split("w4pc", 5120) == wqlib.wq_gemv_max_split("w4g128", 5120)
    tag = "test-w4pc:0"
    wqlib.wq_tune_cache_set("w4pc", 5120, 27648, 1, 0, wqlib.gemv_cache_value(2, 4, 8), tag)
    assert wqlib.wq_tune_cache_get("w4g128", 5120, 27648, 1, 0, tag) == wqlib.gemv_cache_value(2, 4, 8)
    assert wqlib.wq_tune_cache_get("w4pc", 5120, 27648, 1, 0, tag) == wqlib.gemv_cache_value(2, 4, 8)


def test_small_groups_host_side(wqlib):
    """Groups of 32 and 64 (fmts 4..7): canonical sizes as the oracle's, gfx950 sizes
    with one 16-row metadata tile per group, the shape rules (K % 128, N % 8 for W4),
    zeros required for W4, the matrix-core GEMV and the MoE layer refused, the
    remaining GEMV launch options offered as for group-128, and tuner entries of their
    own (not shared with group-128: the kernels fold by another group size)."""
    for fmt in ("w8g32", "w8g64", "w4g32", "w4g64"):
        gs = int(fmt[3:])
        for K, N in ((1024, 1024), (5120, 27648), (13824, 5120), (256, 40)):
            assert wqlib.wq_packed_sizes(fmt, wqlib.CANONICAL, K, N) == OQ.packed_sizes(fmt, K, N), (fmt, K, N)
            q, s, z = wqlib.wq_packed_sizes(fmt, wqlib.GFX950, K, N)
            n16 = -(-N // 16)
            assert q == (K * N if fmt.startswith("w8") else K * N // 2)
            assert s == 2 * n16 * 16 * (K // gs)
            assert z == (8 * n16 * (K // gs) if fmt.startswith("w4") else 0)
        with pytest.raises(wqlib.WqError) as e:
            wqlib.wq_packed_sizes(fmt, wqlib.CANONICAL, 1024 + 64, 64)   # K % 128 != 0
        assert e.value.status == 2
        assert wqlib.wq_gemv_max_split(fmt, 5120) == wqlib.wq_gemv_max_split(fmt[:3] + "128", 5120)
        for M in range(1, 8):
            for rows in (4, 8, 16):
                assert wqlib.wq_gemv_max_waves(fmt, M, rows) == wqlib.wq_gemv_max_waves(fmt[:3] + "128", M, rows)
            for nb in (16, 32, 64):
                assert wqlib.wq_gemv_max_waves(fmt, M, nb | wqlib.GEMV_MFMA) == -1
    L = wqlib.lib
    x, y = C.c_void_p(0x10000), C.c_void_p(0x20000)
    d = wqlib.WqWeightC(wqlib.FMT["w4g32"], wqlib.GFX950, 1024, 64, 0x1000, 0x2000, 0)
    assert L.wq_gemv(C.byref(d), x, 1, y, 1, None, 0, None) == 1          # W4 without zeros
    d = wqlib.WqWeightC(wqlib.FMT["w8g64"], wqlib.GFX950, 1024, 64, 0x1000, 0x2000, 0)
    off = C.c_void_p(0x30000)
    assert L.wq_moe_linear(C.byref(d), 1, x, off, 8, y, 0, None) == 2     # MoE: not for groups of 64
    assert L.wq_gemv_ex(C.byref(d), x, 1, y, 1, 1, 16 | wqlib.GEMV_MFMA, None, 0, None) == 2
    tag = "test-small-groups:0"
    wqlib.wq_tune_cache_set("w4g32", 5120, 27648, 1, 0, wqlib.gemv_cache_value(2, 4, 8), tag)
    assert wqlib.wq_tune_cache_get("w4g32", 5120, 27648, 1, 0, tag) == wqlib.gemv_cache_value(2, 4, 8)
    assert wqlib.wq_tune_cache_get("w4g128", 5120, 27648, 1, 0, tag) is None


def test_activation_type_validation(wqlib):
    """The *_act entry points: an unknown activation type and, for fp16 x, the GEMV's
    matrix-core and prefetch options are refused on the host."""
    L = wqlib.lib
    x, y = C.c_void_p(0x10000), C.c_void_p(0x20000)
    d = wqlib.WqWeightC(wqlib.FMT["w8pc"], wqlib.GFX950, 1024, 64, 0x1000, 0x2000, 0)
    assert wqlib.ACT == {"bf16": 0, "f16": 1}
    assert L.wq_linear_act(C.byref(d), 2, x, 1, y, None, 0, None) == 1
    assert L.wq_gemv_act(C.byref(d), -1, x, 1, y, 1, 0, 0, None, 0, None) == 1
    assert L.wq_gemm_act(C.byref(d), 7, x, 8, y, 2, None, 0, None) == 1
    assert L.wq_gemv_act(C.byref(d), 1, x, 1, y, 1, 1, 16 | wqlib.GEMV_MFMA, None, 0, None) == 2
    assert L.wq_gemv_act(C.byref(d), 1, x, 1, y, 1, 1, 4 | wqlib.GEMV_PREFETCH, None, 0, None) == 2
    assert L.wq_gemv_act(C.byref(d), 1, x, 1, y, 0, 2, 0, None, 0, None) == 1    # waves without a split
    assert L.wq_gemv_act(C.byref(d), 1, x, 8, y, 1, 0, 0, None, 0, None) == 1    # M > 7


def test_residual_validation(wqlib):
    """The residual entry points refuse a NULL residual and a residual that overlaps y
    without being y, on the host."""
    L = wqlib.lib
    x, y = C.c_void_p(0x10000), C.c_void_p(0x20000)
    d = wqlib.WqWeightC(wqlib.FMT["w8pc"], wqlib.GFX950, 1024, 64, 0x1000, 0x2000, 0)
    assert L.wq_linear_residual(C.byref(d), 0, x, 1, None, y, None, 0, None) == 1
    assert L.wq_linear_residual(C.byref(d), 0, x, 1, C.c_void_p(0x20002), y, None, 0, None) == 1
    assert L.wq_linear_residual(C.byref(d), 0, x, 1, C.c_void_p(0x20001), y, None, 0, None) == 3
    assert L.wq_gemm_residual(C.byref(d), 0, x, 8, C.c_void_p(0x1FFFE), y, 2, None, 0, None) == 1
    assert L.wq_gemv_residual(C.byref(d), 0, x, 1, None, y, 1, 0, 0, None, 0, None) == 1
    assert L.wq_gemv_residual(C.byref(d), 0, x, 1, y, y, 0, 2, 0, None, 0, None) == 1   # waves without split
    assert L.wq_linear_residual(C.byref(d), 5, x, 1, y, y, None, 0, None) == 1          # unknown act
