// C ABI entry points: validation, workspace sizing, the GEMV/GEMM dispatch and the
// split-K / tile tuner with its persisted cache.  Host code only; kernels live in
// the .hip files.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cinttypes>
#include <climits>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <tuple>
#include <vector>

#include "wq_internal.h"

namespace wq {
namespace {
thread_local std::string g_err;

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }
bool pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

struct Key {
  std::string tag;
  int fmt;
  int64_t K, N, M;
  int kind;
  bool operator<(const Key& o) const {
    return std::tie(tag, fmt, K, N, M, kind) < std::tie(o.tag, o.fmt, o.K, o.N, o.M, o.kind);
  }
};
std::mutex g_cache_mu;
std::map<Key, int> g_cache;

std::mutex g_dev_mu;
std::map<int, std::string> g_dev_tags;

int64_t split_units(const wq_weight* w) { return gemv_slices(w->K, w->fmt); }

// Largest power of two <= min(v, units, 32).
int clamp_split(int v, int64_t units) {
  int s = 1;
  while (s * 2 <= v && s * 2 <= units && s * 2 <= kMaxSplit) s *= 2;
  return s;
}

// Untuned defaults.  The awq heuristic page starts from split_k = 8 on its GPUs; here
// the workgroup's own waves already split K (no second launch, no workspace), so one
// cross-workgroup slice is the default and split_k > 1 is left to the tuner.
constexpr int kDefaultSplit = 1;
constexpr int kDefaultTile = 9;
static_assert(WQ_GEMM_TILES <= WQ_TUNE_LAT_SLOTS && 6 <= WQ_TUNE_LAT_SLOTS,
              "wq_tune writes one lat_us slot per GEMM tile or GEMV split");

// Tuned GEMV choice: split_k in bits 0..7, waves per workgroup in bits 8..15, rows per
// wave in bits 16..23 (0 = the default for the shape), the slice-prefetch flag in bit
// 24 and the matrix-core flag in bit 25 (rows | WQ_GEMV_PREFETCH / WQ_GEMV_MFMA,
// shifted like rows).
int gemv_value(int split, int waves, int rows) { return split | (waves << 8) | (rows << 16); }
// rows argument of the GEMV: 0, 4, 8 or 16 (optionally | prefetch) or 16 NB | mfma
bool valid_gemv_rows(int rows) {
  if (rows & kGemvMfma) {
    const int rr = rows & ~kGemvMfma;
    return rr == 16 || rr == 32 || rr == 64;
  }
  const int rr = rows & ~kGemvPrefetch;
  return (rr == 0 || rr == 4 || rr == 8 || rr == 16) && !((rows & kGemvPrefetch) && rr == 0);
}
bool valid_gemv_value(int v) {
  const int split = v & 0xFF, waves = (v >> 8) & 0xFF;
  return (v >> 26) == 0 && pow2(split) && split <= kMaxSplit && waves <= kGemvMaxWaves &&
         valid_gemv_rows((v >> 16) & (0xFF | kGemvPrefetch | kGemvMfma));
}

std::string resolve_tag(const char* tag) {
  if (tag && tag[0]) return std::string(tag);
  return current_device_tag();
}

bool cache_lookup(const std::string& tag, int fmt, int64_t K, int64_t N, int64_t M, int kind,
                  int* v) {
  std::lock_guard<std::mutex> lk(g_cache_mu);
  auto it = g_cache.find(Key{tag, fmt, K, N, M, kind});
  if (it == g_cache.end()) return false;
  *v = it->second;
  return true;
}

wq_status check_gemv_split(const wq_weight* w, int M, int split, void* ws, size_t ws_bytes) {
  const int64_t units = split_units(w);
  if (!pow2(split) || split > kMaxSplit || split > units)
    return fail(WQ_ERR_INVALID_ARG, "split_k must be a power of two <= " +
                                        std::to_string(clamp_split(kMaxSplit, units)) + " for this K");
  if (split > 1) {
    if (!ws) return fail(WQ_ERR_WORKSPACE, "split_k > 1 needs a workspace");
    if (!aligned(ws, 16)) return fail(WQ_ERR_ALIGNMENT, "workspace must be 16-byte aligned");
    if (ws_bytes < gemv_workspace_bytes(w->N, M, split))
      return fail(WQ_ERR_WORKSPACE, "workspace too small: need " +
                                        std::to_string(gemv_workspace_bytes(w->N, M, split)) + " bytes");
  }
  return WQ_OK;
}

wq_status check_xy(const void* x, const void* y, int64_t M) {
  if (M < 1) return fail(WQ_ERR_INVALID_ARG, "M must be >= 1");
  if (!x || !y) return fail(WQ_ERR_INVALID_ARG, "x and y must not be NULL");
  if (!aligned(x, 16)) return fail(WQ_ERR_ALIGNMENT, "x must be 16-byte aligned");
  if (!aligned(y, 2)) return fail(WQ_ERR_ALIGNMENT, "y must be 2-byte aligned");
  return WQ_OK;
}

// Tuned (split_k, waves, rows) for this shape, or the defaults (0 = default).
void resolve_gemv(const wq_weight* w, int64_t M, int* split, int* waves, int* rows) {
  int v = 0;
  if (cache_lookup(current_device_tag(), w->fmt, w->K, w->N, M, WQ_KIND_GEMV, &v)) {
    *split = v & 0xFF;
    *waves = (v >> 8) & 0xFF;
    *rows = (v >> 16) & (0xFF | kGemvPrefetch | kGemvMfma);
    return;
  }
  *split = clamp_split(kDefaultSplit, split_units(w));
  *waves = 0;
  *rows = 0;
}

// Untuned GEMM tile: up to 16 tokens the matrix-core GEMV tiles (uint4, and int8 on the
// smaller shapes) or the skinny kernel, with the smallest split-K that gives about two
// workgroups per CU; 17..128 tokens the 64-row LDS-DMA tiles (14..16); 129..256 the
// 128-row ones (17..19); above that the 8-wave LDS-DMA kernel (tile 9) for every format,
// split over K (tiles 10..12, 24) when its tiles are fewer than the CUs, or with its
// partial last round split over K (tile 13).
int default_tile(const wq_weight* w, int64_t M) {
  if (M > 16 && M <= kSkinnyMaxM && w->K % 64 == 0) {
    // 64-row LDS-DMA tiles: the smallest split-K that gives at least 0.6 workgroups per
    // CU (measured on MI355X at M = 32..128: they beat the skinny kernel by 10-37 %; at
    // N = 5120 split 8 (160 workgroups) beats 16 (320: a second, partial round) -- int8
    // at M = 64 31 against 41 us, uint4 45 against 58 us)
    const int64_t blocks = ((M + 63) / 64) * ((w->N + 255) / 256);
    const int64_t want = 3 * (int64_t)device_cus() / 5;
    static constexpr int kSplits64[] = {kDma64Tile0, kDma64Tile0 + 1, kDma64TileLast, kDma64DeepTile0,
                                        kDma64DeepTileLast};  // split-K 1, 2, 4, 8, 16
    int i = 0;
    while (i + 1 < 5 && blocks * gemm_dma64_split(kSplits64[i], M, w->N) < want &&
           gemm_dma64_split(kSplits64[i + 1], M, w->N) > gemm_dma64_split(kSplits64[i], M, w->N))
      ++i;
    return kSplits64[i];
  }
  if (M > kSkinnyMaxM && M <= 2 * kSkinnyMaxM && w->K % 64 == 0) {
    // 128-row LDS-DMA tiles, the same rule (measured on MI355X at M = 256: 12 % faster
    // than the 256-row tiles with or without split-K on the decode projection shapes)
    const int64_t blocks = ((M + 127) / 128) * ((w->N + 255) / 256);
    static constexpr int kSplits128[] = {kDma128Tile0, kDma128Tile0 + 1, kDma128TileLast, kDma128DeepTile0,
                                         kDma128DeepTileLast};  // split-K 1, 2, 4, 8, 16
    int i = 0;
    while (i + 1 < 5 && blocks * gemm_dma64_split(kSplits128[i], M, w->N) < 200 &&
           gemm_dma64_split(kSplits128[i + 1], M, w->N) > gemm_dma64_split(kSplits128[i], M, w->N))
      ++i;
    return kSplits128[i];
  }
  if (M <= kMmaTokens) {
    // measured on MI355X at M = 8..16: uint4 (5120, 27648) 23.6 us with 64 rows per
    // workgroup against 42.6 us for the best skinny tile, (13824, 5120) 19.0 us with 32
    // against 30.8 us; int8 (5120, 7168) 12.5 us against 13.8 us up to 12 tokens, while
    // the skinny kernel stays ahead for int8 on wide N or long K
    if (w->fmt == WQ_FMT_W4_G128) return w->N >= 16384 ? kMmaTile0 + 2 : kMmaTile0 + 1;
    if (small_group(w->fmt)) return kDma64Tile0;  // no matrix-core GEMV or skinny tile for them
    if (w->N < 16384 && w->K < 8192 && M <= 12) return kMmaTile0 + 1;
  }
  if (M <= kSkinnyMaxM && small_group(w->fmt)) return kDma64Tile0;
  if (M <= kSkinnyMaxM) {
    const int64_t blocks = (w->N + 127) / 128;
    int t = kSkinnyTile0;
    while (t < kSkinnyTileLast && blocks * gemm_skinny_split(t, M, w->N) < 512 &&
           gemm_skinny_split(t + 1, M, w->N) > gemm_skinny_split(t, M, w->N))
      ++t;
    return t;
  }
  // fewer tiles (256 x 256 for per-channel W8, 128 x 256 for group-128) than CUs: the
  // split-K (2, 3, 4 or 8; tiles 10, 24, 11, 12) whose rounds of workgroups per unit of
  // work are fewest, ties to the smaller split (measured on MI355X at N = 5120: 40 tiles
  // run best split 4, 80 and 160 group-128 tiles split 3 -- 107 against 139 us and 207
  // against 239 us for uint4 at M = 512 and 1024 -- and 80 per-channel tiles split 3)
  const int64_t tm = gemm_big_dma_rows(w->fmt);
  const int64_t blocks = ((M + tm - 1) / tm) * ((w->N + 255) / 256);
  const int64_t cus = device_cus();
  if (blocks < cus) {
    int best_t = kDefaultTile;
    double best = 1.0;  // unsplit: one round
    for (const int t : {kDmaSplitTile0, kDmaSplit3Tile, kDmaSplitTile0 + 1, kDmaSplitTileLast}) {
      const int S = gemm_dma_split(w->fmt, t, M, w->N);
      if (S <= 1) continue;
      const double r = (double)((blocks * S + cus - 1) / cus) / S;
      if (r < best - 1e-9) {
        best = r;
        best_t = t;
      }
    }
    return best_t;
  }
  // a partial last round of tiles that would leave at least half the CUs idle: tile 13
  // spreads it over K (it needs a workspace; without one it runs as tile 9)
  int tail0 = 0;
  return gemm_dma_tail(w->fmt, M, w->N, &tail0) > 1 ? kDmaTailTile : kDefaultTile;
}

int resolve_tile(const wq_weight* w, int64_t M) {
  int v = 0;
  if (!cache_lookup(current_device_tag(), w->fmt, w->K, w->N, M, WQ_KIND_GEMM, &v)) v = default_tile(w, M);
  return small_group(w->fmt) ? small_group_tile(v) : v;
}

wq_status gemv_impl(const wq_weight* w0, const void* x, int64_t M, void* y, int split_k, int waves,
                    int rows, void* ws, size_t ws_bytes, void* stream, int act = WQ_ACT_BF16,
                    const void* res = nullptr) {
  if (act != WQ_ACT_BF16 && act != WQ_ACT_F16) return fail(WQ_ERR_INVALID_ARG, "unknown activation type");
  const bool xf = act == WQ_ACT_F16;
  wq_status st = check_weight(w0, WQ_LAYOUT_GFX950);
  if (st != WQ_OK) return st;
  const wq_weight cview = compute_view(*w0);
  const wq_weight* w = &cview;
  if ((st = check_xy(x, y, M)) != WQ_OK) return st;
  if (M > kGemvMaxM) return fail(WQ_ERR_INVALID_ARG, "wq_gemv: M must be in 1..7");
  if (split_k < 0 || waves < 0 || waves > kGemvMaxWaves)
    return fail(WQ_ERR_INVALID_ARG, "wq_gemv: waves per workgroup must be 0 (default) or 1..16");
  if (!valid_gemv_rows(rows))
    return fail(WQ_ERR_INVALID_ARG,
                "wq_gemv: rows per wave must be 0 (default), 4, 8 or 16 (optionally | WQ_GEMV_PREFETCH), "
                "or 16, 32, 64 or 128 | WQ_GEMV_MFMA");
  if (rows & (kGemvPrefetch | kGemvMfma) && gemv_max_waves(w->fmt, (int)M, rows) == 0)
    return fail(WQ_ERR_UNSUPPORTED, "wq_gemv: this rows flag is not offered at this format, M and rows");
  if (xf && (rows & (kGemvPrefetch | kGemvMfma)))
    return fail(WQ_ERR_UNSUPPORTED, "wq_gemv: fp16 activations take rows 4, 8 or 16 without flags");
  int split = split_k, wv = waves, rw = rows;
  if (split_k == 0) {
    int tw = 0, tr = 0;
    resolve_gemv(w, M, &split, &tw, &tr);
    if (xf && (tr & kGemvMfma)) tw = tr = 0;  // (tuned for bf16 x:) the default dot2 launch
    if (xf) tr &= ~kGemvPrefetch;             // the same launch without the prefetch set
    if (wv == 0) wv = tw;
    if (rw == 0) rw = tr;
    if (split > 1 && (!ws || ws_bytes < gemv_workspace_bytes(w->N, M, split))) {
      split = 1;  // the tuned split needs more workspace than given: one slice range
      wv = 0;
    }
  }
  if ((st = check_gemv_split(w, (int)M, split, ws, ws_bytes)) != WQ_OK) return st;
  if (rw == 0) rw = gemv_default_rows(w->K, w->N, w->fmt, (int)M);
  if (wv == 0) wv = gemv_default_waves(w->K, w->N, w->fmt, (int)M, split, rw);
  return launch_gemv(w, (const uint16_t*)x, (int)M, (uint16_t*)y, split, wv, rw, ws,
                     (hipStream_t)stream, xf, (const uint16_t*)res);
}

wq_status gemm_impl(const wq_weight* w0, const void* x, int64_t M, void* y, int tile, void* ws,
                    size_t ws_bytes, void* stream, int act = WQ_ACT_BF16, const void* res = nullptr) {
  if (act != WQ_ACT_BF16 && act != WQ_ACT_F16) return fail(WQ_ERR_INVALID_ARG, "unknown activation type");
  const bool xf = act == WQ_ACT_F16;
  wq_status st = check_weight(w0, WQ_LAYOUT_GFX950);
  if (st != WQ_OK) return st;
  const wq_weight cview = compute_view(*w0);
  const wq_weight* w = &cview;
  if ((st = check_xy(x, y, M)) != WQ_OK) return st;
  if (tile < 0 || tile > WQ_GEMM_TILES) return fail(WQ_ERR_INVALID_ARG, "wq_gemm: bad tile id");
  int t = tile == 0 ? resolve_tile(w, M) : small_group(w->fmt) ? small_group_tile(tile) : tile;
  if (xf) t = act_tile(w->fmt, t);
  if (tile != 0 && gemm_workspace_bytes(w->fmt, w->N, M, t) > 0 && (!ws || ws_bytes < gemm_workspace_bytes(w->fmt, w->N, M, t)))
    return fail(WQ_ERR_WORKSPACE, "wq_gemm: tile " + std::to_string(t) + " needs a workspace of " +
                                      std::to_string(gemm_workspace_bytes(w->fmt, w->N, M, t)) + " bytes");
  return launch_gemm(w, (const uint16_t*)x, M, (uint16_t*)y, t, ws, ws_bytes, (hipStream_t)stream, xf,
                     (const uint16_t*)res);
}

}  // namespace

void set_error(const std::string& msg) { g_err = msg; }
wq_status fail(wq_status st, const std::string& msg) {
  g_err = msg;
  return st;
}
wq_status hip_fail(hipError_t e, const char* what) {
  g_err = std::string(what) + ": " + hipGetErrorString(e);
  return (e == hipErrorNoDevice || e == hipErrorInvalidDevice) ? WQ_ERR_NO_DEVICE : WQ_ERR_HIP;
}

std::string current_device_tag() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return std::string();
  std::lock_guard<std::mutex> lk(g_dev_mu);
  auto it = g_dev_tags.find(dev);
  if (it != g_dev_tags.end()) return it->second;
  hipDeviceProp_t p;
  if (hipGetDeviceProperties(&p, dev) != hipSuccess) return std::string();
  std::string arch(p.gcnArchName);
  const size_t colon = arch.find(':');
  if (colon != std::string::npos) arch.resize(colon);
  std::string tag = arch + ":" + std::to_string(p.multiProcessorCount);
  g_dev_tags[dev] = tag;
  return tag;
}

wq_status check_shape(int fmt, int64_t K, int64_t N) {
  if (fmt < WQ_FMT_W8_PC || fmt > WQ_FMT_W4_G64) return fail(WQ_ERR_UNSUPPORTED, "unknown format");
  if (K <= 0 || N <= 0) return fail(WQ_ERR_INVALID_ARG, "K and N must be positive");
  if (K > (1LL << 22) || N > (1LL << 30)) return fail(WQ_ERR_UNSUPPORTED, "K or N too large");
  if (K % 16) return fail(WQ_ERR_UNSUPPORTED, "K must be a multiple of 16");
  if (fmt != WQ_FMT_W8_PC && K % kGroup)
    return fail(WQ_ERR_UNSUPPORTED, "grouped formats and W4 per channel need K % 128 == 0");
  if (is_w4(fmt) && N % 8) return fail(WQ_ERR_UNSUPPORTED, "W4 needs N % 8 == 0");
  return WQ_OK;
}

wq_status check_weight(const wq_weight* w, int want_layout) {
  if (!w) return fail(WQ_ERR_INVALID_ARG, "weight descriptor is NULL");
  wq_status st = check_shape(w->fmt, w->K, w->N);
  if (st != WQ_OK) return st;
  if (w->layout != want_layout)
    return fail(WQ_ERR_UNSUPPORTED, want_layout == WQ_LAYOUT_GFX950
                                        ? "compute kernels need the GFX950 layout (call wq_repack)"
                                        : "expected the CANONICAL layout");
  if (!w->qweight || !w->scales) return fail(WQ_ERR_INVALID_ARG, "qweight/scales must not be NULL");
  if (is_w4(w->fmt) && !w->zeros) return fail(WQ_ERR_INVALID_ARG, "W4 needs zeros");
  if (!aligned(w->qweight, 16)) return fail(WQ_ERR_ALIGNMENT, "qweight must be 16-byte aligned");
  if (!aligned(w->scales, want_layout == WQ_LAYOUT_GFX950 && w->fmt != WQ_FMT_W8_PC ? 16 : 2))
    return fail(WQ_ERR_ALIGNMENT, "scales must be 2-byte aligned (16-byte for tiled gfx950 scales)");
  if (is_w4(w->fmt) && want_layout == WQ_LAYOUT_GFX950 && !aligned(w->zeros, 8))
    return fail(WQ_ERR_ALIGNMENT, "gfx950 zeros must be 8-byte aligned");
  if (is_w4(w->fmt) && want_layout == WQ_LAYOUT_CANONICAL && !aligned(w->zeros, 4))
    return fail(WQ_ERR_ALIGNMENT, "canonical zeros must be 4-byte aligned");
  return WQ_OK;
}

}  // namespace wq

using namespace wq;

extern "C" {

int wq_abi_version(void) { return WQ_ABI_VERSION; }

const char* wq_status_string(int s) {
  switch (s) {
    case WQ_OK: return "ok";
    case WQ_ERR_INVALID_ARG: return "invalid argument";
    case WQ_ERR_UNSUPPORTED: return "unsupported format, layout or shape";
    case WQ_ERR_ALIGNMENT: return "misaligned pointer";
    case WQ_ERR_WORKSPACE: return "workspace missing or too small";
    case WQ_ERR_NO_DEVICE: return "no HIP device";
    case WQ_ERR_HIP: return "HIP runtime error";
    case WQ_ERR_CACHE_IO: return "tuner cache I/O error";
  }
  return "unknown status";
}

const char* wq_last_error(void) { return g_err.c_str(); }

wq_status wq_packed_sizes(int fmt, int layout, int64_t K, int64_t N, size_t* qb, size_t* sb,
                          size_t* zb) {
  wq_status st = check_shape(fmt, K, N);
  if (st != WQ_OK) return st;
  if (layout != WQ_LAYOUT_CANONICAL && layout != WQ_LAYOUT_GFX950)
    return fail(WQ_ERR_UNSUPPORTED, "unknown layout");
  const int64_t G = fmt == WQ_FMT_W8_PC ? 0 : K / meta_group(fmt);  // groups per row (gfx950 metadata)
  size_t q = 0, s = 0, z = 0;
  switch (fmt) {
    case WQ_FMT_W8_PC: q = (size_t)(K * N); s = (size_t)(2 * N); break;
    case WQ_FMT_W8_G32:
    case WQ_FMT_W8_G64:
    case WQ_FMT_W8_G128:
      q = (size_t)(K * N);
      s = layout == WQ_LAYOUT_CANONICAL ? (size_t)(2 * N * G) : (size_t)(2 * row_tiles(N) * G * kGemvTileRows);
      break;
    case WQ_FMT_W4_G32:
    case WQ_FMT_W4_G64:
    case WQ_FMT_W4_G128:
    case WQ_FMT_W4_PC: {
      // per channel: one group in the canonical layout, K/128 repeated ones in gfx950's
      const int64_t Gc = fmt == WQ_FMT_W4_PC ? 1 : G;
      q = (size_t)(K * N / 2);
      s = layout == WQ_LAYOUT_CANONICAL ? (size_t)(2 * N * Gc) : (size_t)(2 * row_tiles(N) * G * kGemvTileRows);
      z = layout == WQ_LAYOUT_CANONICAL ? (size_t)(Gc * (N / 8) * 4)
                                        : (size_t)(row_tiles(N) * G * (kGemvTileRows / 2));
      break;
    }
  }
  if (qb) *qb = q;
  if (sb) *sb = s;
  if (zb) *zb = z;
  return WQ_OK;
}

int wq_gemv_max_split(int fmt, int64_t K) {
  if (check_shape(fmt, K, 8) != WQ_OK) return -1;
  return clamp_split(kMaxSplit, gemv_slices(K, compute_fmt(fmt)));
}

int wq_gemv_max_waves(int fmt, int64_t M, int rows) {
  if (fmt < WQ_FMT_W8_PC || fmt > WQ_FMT_W4_G64 || M < 1 || M > kGemvMaxM) return -1;
  const int cap = gemv_max_waves(compute_fmt(fmt), (int)M, rows);
  return cap > 0 ? cap : -1;
}

int wq_dispatch_kind(int64_t M) {
  if (M < 1) return -1;
  return M <= kGemvMaxM ? WQ_KIND_GEMV : WQ_KIND_GEMM;
}

wq_status wq_pack(const float* w, const wq_weight* out, void* stream) {
  wq_status st = check_weight(out, WQ_LAYOUT_CANONICAL);
  if (st != WQ_OK) return st;
  if (!w) return fail(WQ_ERR_INVALID_ARG, "w must not be NULL");
  if (!aligned(w, 16)) return fail(WQ_ERR_ALIGNMENT, "w must be 16-byte aligned");
  return launch_pack(w, out, (hipStream_t)stream);
}

wq_status wq_pack_bf16(const void* w, const wq_weight* out, void* stream) {
  wq_status st = check_weight(out, WQ_LAYOUT_CANONICAL);
  if (st != WQ_OK) return st;
  if (!w) return fail(WQ_ERR_INVALID_ARG, "w must not be NULL");
  if (!aligned(w, 8)) return fail(WQ_ERR_ALIGNMENT, "w (bf16) must be 8-byte aligned");
  return launch_pack_bf16((const uint16_t*)w, out, (hipStream_t)stream);
}

static wq_status repack_common(const wq_weight* src, const wq_weight* dst, int from, int to,
                               void* stream) {
  wq_status st = check_weight(src, from);
  if (st != WQ_OK) return st;
  if ((st = check_weight(dst, to)) != WQ_OK) return st;
  if (src->fmt != dst->fmt || src->K != dst->K || src->N != dst->N)
    return fail(WQ_ERR_INVALID_ARG, "src and dst differ in format or shape");
  if (src->qweight == dst->qweight || src->scales == dst->scales ||
      (src->zeros && src->zeros == dst->zeros))
    return fail(WQ_ERR_INVALID_ARG, "repack cannot run in place");
  return launch_repack(src, dst, to == WQ_LAYOUT_GFX950, (hipStream_t)stream);
}

wq_status wq_repack(const wq_weight* src, const wq_weight* dst, void* stream) {
  return repack_common(src, dst, WQ_LAYOUT_CANONICAL, WQ_LAYOUT_GFX950, stream);
}

wq_status wq_unrepack(const wq_weight* src, const wq_weight* dst, void* stream) {
  return repack_common(src, dst, WQ_LAYOUT_GFX950, WQ_LAYOUT_CANONICAL, stream);
}

wq_status wq_workspace_size(const wq_weight* w0, int64_t M, size_t* bytes) {
  if (!w0 || !bytes) return fail(WQ_ERR_INVALID_ARG, "NULL argument");
  wq_status st = check_shape(w0->fmt, w0->K, w0->N);
  if (st != WQ_OK) return st;
  const wq_weight cview = compute_view(*w0);
  const wq_weight* w = &cview;
  if (M < 1) return fail(WQ_ERR_INVALID_ARG, "M must be >= 1");
  if (M <= kGemvMaxM) {
    *bytes = gemv_workspace_bytes(w->N, M, kMaxSplit);
  } else {
    size_t b = 0;
    for (int t = 1; t <= WQ_GEMM_TILES; ++t)
      if (!small_group(w->fmt) || small_group_tile(t) == t)
        b = std::max(b, gemm_workspace_full_bytes(w->fmt, w->K, w->N, M, t));
    *bytes = b;
  }
  return WQ_OK;
}

wq_status wq_gemv(const wq_weight* w, const void* x, int64_t M, void* y, int split_k, void* ws,
                  size_t ws_bytes, void* stream) {
  return gemv_impl(w, x, M, y, split_k, 0, 0, ws, ws_bytes, stream);
}

wq_status wq_gemv_ex(const wq_weight* w, const void* x, int64_t M, void* y, int split_k, int waves,
                     int rows, void* ws, size_t ws_bytes, void* stream) {
  if (split_k < 1) return fail(WQ_ERR_INVALID_ARG, "wq_gemv_ex: split_k must be given (>= 1)");
  return gemv_impl(w, x, M, y, split_k, waves, rows, ws, ws_bytes, stream);
}

wq_status wq_gemm(const wq_weight* w, const void* x, int64_t M, void* y, int tile, void* ws,
                  size_t ws_bytes, void* stream) {
  return gemm_impl(w, x, M, y, tile, ws, ws_bytes, stream);
}

wq_status wq_linear(const wq_weight* w, const void* x, int64_t M, void* y, void* ws, size_t ws_bytes,
                    void* stream) {
  if (M < 1) return fail(WQ_ERR_INVALID_ARG, "M must be >= 1");
  if (wq_dispatch_kind(M) == WQ_KIND_GEMV) return gemv_impl(w, x, M, y, 0, 0, 0, ws, ws_bytes, stream);
  return gemm_impl(w, x, M, y, 0, ws, ws_bytes, stream);
}

wq_status wq_linear_act(const wq_weight* w, int act, const void* x, int64_t M, void* y, void* ws,
                        size_t ws_bytes, void* stream) {
  if (M < 1) return fail(WQ_ERR_INVALID_ARG, "M must be >= 1");
  if (wq_dispatch_kind(M) == WQ_KIND_GEMV) return gemv_impl(w, x, M, y, 0, 0, 0, ws, ws_bytes, stream, act);
  return gemm_impl(w, x, M, y, 0, ws, ws_bytes, stream, act);
}

wq_status wq_gemv_act(const wq_weight* w, int act, const void* x, int64_t M, void* y, int split_k, int waves,
                      int rows, void* ws, size_t ws_bytes, void* stream) {
  if (split_k < 0) return fail(WQ_ERR_INVALID_ARG, "wq_gemv_act: split_k must be 0 (tuned) or >= 1");
  if (split_k == 0 && (waves != 0 || rows != 0))
    return fail(WQ_ERR_INVALID_ARG, "wq_gemv_act: waves and rows need an explicit split_k");
  return gemv_impl(w, x, M, y, split_k, waves, rows, ws, ws_bytes, stream, act);
}

wq_status wq_gemm_act(const wq_weight* w, int act, const void* x, int64_t M, void* y, int tile, void* ws,
                      size_t ws_bytes, void* stream) {
  return gemm_impl(w, x, M, y, tile, ws, ws_bytes, stream, act);
}

wq_status wq_linear_residual(const wq_weight* w, int act, const void* x, int64_t M, const void* r, void* y,
                             void* ws, size_t ws_bytes, void* stream) {
  if (M < 1) return fail(WQ_ERR_INVALID_ARG, "M must be >= 1");
  if (!r) return fail(WQ_ERR_INVALID_ARG, "wq_linear_residual: NULL residual");
  if (!aligned(r, 2)) return fail(WQ_ERR_ALIGNMENT, "wq_linear_residual: the residual needs 2-byte alignment");
  if (r != y && w && (const char*)r < (const char*)y + (size_t)M * w->N * 2 &&
      (const char*)y < (const char*)r + (size_t)M * w->N * 2)
    return fail(WQ_ERR_INVALID_ARG, "wq_linear_residual: the residual overlaps y without being y");
  if (wq_dispatch_kind(M) == WQ_KIND_GEMV) return gemv_impl(w, x, M, y, 0, 0, 0, ws, ws_bytes, stream, act, r);
  return gemm_impl(w, x, M, y, 0, ws, ws_bytes, stream, act, r);
}

wq_status wq_gemm_residual(const wq_weight* w, int act, const void* x, int64_t M, const void* r, void* y, int tile,
                           void* ws, size_t ws_bytes, void* stream) {
  if (!r) return fail(WQ_ERR_INVALID_ARG, "wq_gemm_residual: NULL residual");
  if (!aligned(r, 2)) return fail(WQ_ERR_ALIGNMENT, "wq_gemm_residual: the residual needs 2-byte alignment");
  if (r != y && w && (const char*)r < (const char*)y + (size_t)M * w->N * 2 &&
      (const char*)y < (const char*)r + (size_t)M * w->N * 2)
    return fail(WQ_ERR_INVALID_ARG, "wq_gemm_residual: the residual overlaps y without being y");
  return gemm_impl(w, x, M, y, tile, ws, ws_bytes, stream, act, r);
}

wq_status wq_gemv_residual(const wq_weight* w, int act, const void* x, int64_t M, const void* r, void* y,
                           int split_k, int waves, int rows, void* ws, size_t ws_bytes, void* stream) {
  if (!r) return fail(WQ_ERR_INVALID_ARG, "wq_gemv_residual: NULL residual");
  if (!aligned(r, 2)) return fail(WQ_ERR_ALIGNMENT, "wq_gemv_residual: the residual needs 2-byte alignment");
  if (r != y && w && (const char*)r < (const char*)y + (size_t)M * w->N * 2 &&
      (const char*)y < (const char*)r + (size_t)M * w->N * 2)
    return fail(WQ_ERR_INVALID_ARG, "wq_gemv_residual: the residual overlaps y without being y");
  if (split_k < 0 || (split_k == 0 && (waves != 0 || rows != 0)))
    return fail(WQ_ERR_INVALID_ARG, "wq_gemv_residual: split_k 0 (tuned, with waves = rows = 0) or >= 1");
  return gemv_impl(w, x, M, y, split_k, waves, rows, ws, ws_bytes, stream, act, r);
}

// ------------------------------------------------- the layer without allocation
namespace {
// Scratch of wq_linear_static: one copy per device, held from the library's load to
// the end of the process.  In host code `scratch` names a host-side stand-in of the
// symbol, never the device memory: kernels get the per-device address that
// hipGetSymbolAddress returns for it (static_scratch below), nothing else.
__device__ __align__(256) uint8_t scratch[WQ_STATIC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
std::map<int, void*> g_scratch_ptr;

// Device address of this device's scratch (looked up once per device, with that device
// current), or NULL with the error text set.
void* static_scratch(wq_status* st) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *st = hip_fail(e, "hipGetDevice");
    return nullptr;
  }
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  auto it = g_scratch_ptr.find(dev);
  if (it != g_scratch_ptr.end()) return it->second;
  void* ptr = nullptr;
  e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !ptr) {
    *st = e != hipSuccess ? hip_fail(e, "hipGetSymbolAddress(scratch)")
                          : fail(WQ_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    return nullptr;
  }
  g_scratch_ptr[dev] = ptr;
  return ptr;
}
}  // namespace

wq_status wq_linear_static(const wq_weight* w0, const void* x, int64_t M, void* y, void* stream) {
  if (M < 1) return fail(WQ_ERR_INVALID_ARG, "M must be >= 1");
  wq_status st = check_weight(w0, WQ_LAYOUT_GFX950);
  if (st != WQ_OK) return st;
  const wq_weight cview = compute_view(*w0);
  const wq_weight* w = &cview;
  // the workspace the configuration wq_linear would run needs (its split-K partials)
  size_t need = 0;
  if (wq_dispatch_kind(M) == WQ_KIND_GEMV) {
    int split = 1, waves = 0, rows = 0;
    resolve_gemv(w, M, &split, &waves, &rows);
    need = gemv_workspace_bytes(w->N, M, split);
  } else {
    need = gemm_workspace_bytes(w->fmt, w->N, M, resolve_tile(w, M));
  }
  if (need > (size_t)WQ_STATIC_SCRATCH_BYTES)
    return fail(WQ_ERR_WORKSPACE, "wq_linear_static: this shape's configuration needs " + std::to_string(need) +
                                      " bytes of partial sums, more than the " +
                                      std::to_string((size_t)WQ_STATIC_SCRATCH_BYTES) +
                                      "-byte static scratch; call wq_linear with a workspace");
  void* ws = static_scratch(&st);
  if (!ws) return st;
  return wq_linear(w, x, M, y, ws, (size_t)WQ_STATIC_SCRATCH_BYTES, stream);
}

// ------------------------------------------------------- grouped (MoE) layer
wq_status wq_moe_linear(const wq_weight* w0, int E, const void* x, const int32_t* offsets, int64_t T, void* y,
                        int epilogue, void* stream) {
  wq_status st = check_weight(w0, WQ_LAYOUT_GFX950);
  if (st != WQ_OK) return st;
  const wq_weight cview = compute_view(*w0);
  const wq_weight* w = &cview;
  if (E < 1 || E > 65535) return fail(WQ_ERR_INVALID_ARG, "wq_moe_linear: E must lie in 1 .. 65535");
  if (T < 0 || T > INT32_MAX) return fail(WQ_ERR_INVALID_ARG, "wq_moe_linear: T must lie in 0 .. 2^31 - 1");
  if (epilogue != WQ_EPILOGUE_NONE && epilogue != WQ_EPILOGUE_SILU_MUL)
    return fail(WQ_ERR_INVALID_ARG, "wq_moe_linear: unknown epilogue");
  if (!x || !y || !offsets) return fail(WQ_ERR_INVALID_ARG, "NULL argument");
  if (!aligned(x, 16) || !aligned(y, 2) || !aligned(offsets, 4))
    return fail(WQ_ERR_ALIGNMENT, "wq_moe_linear: x needs 16-byte, y 2-byte and offsets 4-byte alignment");
  if (small_group(w->fmt))
    return fail(WQ_ERR_UNSUPPORTED, "wq_moe_linear: takes per-channel and group-128 formats");
  if (w->K % kGroup != 0 || w->N % 16 != 0 || (epilogue == WQ_EPILOGUE_SILU_MUL && w->N % 32 != 0))
    return fail(WQ_ERR_UNSUPPORTED,
                "wq_moe_linear: needs K % 128 == 0 and N % 16 == 0 (N % 32 == 0 with the gated epilogue)");
  if (T * w->K >= (int64_t(1) << 31) || T * w->N >= (int64_t(1) << 31))
    return fail(WQ_ERR_UNSUPPORTED, "wq_moe_linear: T * K and T * N must stay below 2^31");
  if (T == 0) return WQ_OK;
  size_t qb = 0, sb = 0, zb = 0;
  if ((st = wq_packed_sizes(w->fmt, WQ_LAYOUT_GFX950, w->K, w->N, &qb, &sb, &zb)) != WQ_OK) return st;
  return launch_moe(w, E, (const uint16_t*)x, offsets, T, (uint16_t*)y, epilogue == WQ_EPILOGUE_SILU_MUL, qb, sb,
                    zb, (hipStream_t)stream);
}

// ------------------------------------------------------------ LM head + top-k
namespace {
struct TopkLayout {
  size_t lin, logits_off, cand_off, total;
};
size_t round_up256(size_t b) { return (b + 255) & ~(size_t)255; }
wq_status topk_layout(const wq_weight* w, int64_t M, int k, TopkLayout* L) {
  if (!w) return fail(WQ_ERR_INVALID_ARG, "NULL weight");
  wq_status st = check_shape(w->fmt, w->K, w->N);
  if (st != WQ_OK) return st;
  if (M < 1) return fail(WQ_ERR_INVALID_ARG, "M must be >= 1");
  if (k < 1 || k > kTopkMaxK || k > w->N)
    return fail(WQ_ERR_INVALID_ARG, "wq_lm_head_topk: k must lie in 1 .. min(64, N)");
  if ((int64_t)topk_chunks(w->N) * k > kTopkMergeMax)
    return fail(WQ_ERR_UNSUPPORTED, "wq_lm_head_topk: ceil(N / 2048) * k must not exceed 8192");
  if ((st = wq_workspace_size(w, M, &L->lin)) != WQ_OK) return st;
  L->logits_off = round_up256(L->lin);
  L->cand_off = round_up256(L->logits_off + (size_t)M * w->N * 2);
  L->total = L->cand_off + (size_t)M * topk_chunks(w->N) * k * sizeof(uint64_t);
  return WQ_OK;
}
}  // namespace

wq_status wq_lm_head_topk_workspace_size(const wq_weight* w, int64_t M, int k, size_t* bytes) {
  if (!bytes) return fail(WQ_ERR_INVALID_ARG, "NULL argument");
  TopkLayout L;
  const wq_status st = topk_layout(w, M, k, &L);
  if (st == WQ_OK) *bytes = L.total;
  return st;
}

wq_status wq_lm_head_topk(const wq_weight* w, const void* x, int64_t M, int k, float temperature, const float* u,
                          void* top_vals, int32_t* top_idx, int32_t* tokens, void* ws, size_t ws_bytes,
                          void* stream) {
  wq_status st = check_weight(w, WQ_LAYOUT_GFX950);
  if (st != WQ_OK) return st;
  TopkLayout L;
  if ((st = topk_layout(w, M, k, &L)) != WQ_OK) return st;
  if (!x || !u || !top_vals || !top_idx || !tokens) return fail(WQ_ERR_INVALID_ARG, "NULL argument");
  if (!(temperature >= 0.f) || !std::isfinite(temperature))
    return fail(WQ_ERR_INVALID_ARG, "wq_lm_head_topk: temperature must be finite and >= 0");
  if (((uintptr_t)u | (uintptr_t)top_idx | (uintptr_t)tokens) % 4 || (uintptr_t)top_vals % 2)
    return fail(WQ_ERR_ALIGNMENT, "wq_lm_head_topk: u, top_idx, tokens need 4-byte, top_vals 2-byte alignment");
  if (!ws || ws_bytes < L.total)
    return fail(WQ_ERR_WORKSPACE, "wq_lm_head_topk needs a workspace of " + std::to_string(L.total) + " bytes");
  if ((uintptr_t)ws % 256)
    return fail(WQ_ERR_ALIGNMENT, "wq_lm_head_topk: the workspace must be 256-byte aligned");
  uint8_t* wsb = (uint8_t*)ws;
  uint16_t* logits = (uint16_t*)(wsb + L.logits_off);
  // the layer itself, confined to its own part of the workspace
  void* lin_ws = L.lin ? ws : nullptr;
  st = wq_dispatch_kind(M) == WQ_KIND_GEMV ? gemv_impl(w, x, M, logits, 0, 0, 0, lin_ws, L.lin, stream)
                                          : gemm_impl(w, x, M, logits, 0, lin_ws, L.lin, stream);
  if (st != WQ_OK) return st;
  return launch_topk(logits, M, w->N, k, temperature, u, (uint64_t*)(wsb + L.cand_off), (uint16_t*)top_vals,
                     top_idx, tokens, (hipStream_t)stream);
}

// ------------------------------------------------- full-K activation permutation
namespace {
// workspace: [the layer's own workspace][x' bf16 [M][K]], x' 256-byte aligned
wq_status perm_layout(const wq_weight* w, int64_t M, size_t* lin, size_t* xp_off, size_t* total) {
  if (!w) return fail(WQ_ERR_INVALID_ARG, "NULL weight");
  wq_status st = check_shape(w->fmt, w->K, w->N);
  if (st != WQ_OK) return st;
  if (M < 1) return fail(WQ_ERR_INVALID_ARG, "M must be >= 1");
  if ((st = wq_workspace_size(w, M, lin)) != WQ_OK) return st;
  *xp_off = round_up256(*lin);
  *total = *xp_off + (size_t)M * w->K * 2;
  return WQ_OK;
}
}  // namespace

wq_status wq_linear_perm_workspace_size(const wq_weight* w, int64_t M, size_t* bytes) {
  if (!bytes) return fail(WQ_ERR_INVALID_ARG, "NULL argument");
  size_t lin = 0, off = 0, total = 0;
  const wq_status st = perm_layout(w, M, &lin, &off, &total);
  if (st == WQ_OK) *bytes = total;
  return st;
}

wq_status wq_linear_perm(const wq_weight* w, const void* x, const int32_t* perm, int64_t M, void* y, void* ws,
                         size_t ws_bytes, void* stream) {
  wq_status st = check_weight(w, WQ_LAYOUT_GFX950);
  if (st != WQ_OK) return st;
  size_t lin = 0, off = 0, total = 0;
  if ((st = perm_layout(w, M, &lin, &off, &total)) != WQ_OK) return st;
  if (!x || !perm || !y) return fail(WQ_ERR_INVALID_ARG, "NULL argument");
  if ((uintptr_t)x % 2 || (uintptr_t)perm % 4 || (uintptr_t)y % 2)
    return fail(WQ_ERR_ALIGNMENT, "wq_linear_perm: x and y need 2-byte, perm 4-byte alignment");
  if (!ws || ws_bytes < total)
    return fail(WQ_ERR_WORKSPACE, "wq_linear_perm needs a workspace of " + std::to_string(total) + " bytes");
  if ((uintptr_t)ws % 256) return fail(WQ_ERR_ALIGNMENT, "wq_linear_perm: the workspace must be 256-byte aligned");
  uint16_t* xp = (uint16_t*)((uint8_t*)ws + off);
  if ((st = launch_perm_gather((const uint16_t*)x, perm, xp, M, w->K, (hipStream_t)stream)) != WQ_OK) return st;
  // the layer on the gathered activations, confined to its own part of the workspace
  void* lin_ws = lin ? ws : nullptr;
  return wq_dispatch_kind(M) == WQ_KIND_GEMV ? gemv_impl(w, xp, M, y, 0, 0, 0, lin_ws, lin, stream)
                                             : gemm_impl(w, xp, M, y, 0, lin_ws, lin, stream);
}

int wq_tune_pick(const double* lat, int n) {
  if (!lat || n < 1) return -1;
  int best = -1;
  for (int i = 0; i < n; ++i) {
    if (lat[i] < 0) continue;  // candidate not run
    if (best < 0 || lat[best] >= lat[i]) best = i;
  }
  return best;
}

wq_status wq_tune(const wq_weight* copies0, int n_copies, int64_t M, const void* x, void* y, void* ws,
                  size_t ws_bytes, int warmup, int iters, void* stream, int* chosen, double* lat_us) {
  if (!copies0 || n_copies < 1 || !chosen || iters < 1 || warmup < 0)
    return fail(WQ_ERR_INVALID_ARG, "wq_tune: bad arguments");
  wq_status st;
  for (int i = 0; i < n_copies; ++i) {
    if ((st = check_weight(&copies0[i], WQ_LAYOUT_GFX950)) != WQ_OK) return st;
    if (copies0[i].fmt != copies0[0].fmt || copies0[i].K != copies0[0].K || copies0[i].N != copies0[0].N)
      return fail(WQ_ERR_INVALID_ARG, "wq_tune: copies differ in format or shape");
  }
  std::vector<wq_weight> views(copies0, copies0 + n_copies);  // as the compute kernels take them
  for (wq_weight& v : views) v = compute_view(v);
  const wq_weight* copies = views.data();
  if ((st = check_xy(x, y, M)) != WQ_OK) return st;
  const bool gemv = wq_dispatch_kind(M) == WQ_KIND_GEMV;
  // GEMV candidates: every (split_k, waves) pair; GEMM candidates: the tiles
  struct Cand {
    int split, waves, rows, tile;
  };
  std::vector<Cand> cand;
  if (gemv) {
    const int fmt = copies[0].fmt;
    for (int s = 1; s <= kMaxSplit; s *= 2)
      for (const int rw : {4, 8, 16, 4 | kGemvPrefetch, 8 | kGemvPrefetch, 16 | kGemvPrefetch,
                           16 | kGemvMfma, 32 | kGemvMfma, 64 | kGemvMfma}) {
        const int cap = gemv_max_waves(fmt, (int)M, rw);
        if (cap == 0) continue;  // flag not offered at this format and M
        const int dflt = gemv_default_waves(copies[0].K, copies[0].N, fmt, (int)M, s, rw);
        // K pieces a workgroup's waves share (1 KB slices, or 128-k units for the
        // matrix-core kernel): a count that is the fewest waves giving each wave at most
        // ceil(P / w) pieces spreads them evenly (P = 14: 5 and 7 waves)
        const int64_t P = (rw & kGemvMfma) ? ((copies[0].K + kGroup - 1) / kGroup + s - 1) / s
                                           : (gemv_slices(copies[0].K, fmt) + s - 1) / s;
        auto balanced = [&](int wv) { return wv == 1 || (P + wv - 1) / wv < (P + wv - 2) / (wv - 1); };
        // powers of two, 3 x powers of two, the balanced counts and the default
        for (int wv = 1; wv <= cap; ++wv)
          if (((wv & (wv - 1)) == 0) || ((wv % 3 == 0) && (((wv / 3) & (wv / 3 - 1)) == 0)) || balanced(wv) ||
              wv == dflt)
            cand.push_back({s, wv, rw, 0});
      }
  } else {
    for (int t = 1; t <= WQ_GEMM_TILES; ++t)
      if (!small_group(copies[0].fmt) || small_group_tile(t) == t)  // the others run as one of these
        cand.push_back({0, 0, 0, t});
  }
  hipStream_t hs = (hipStream_t)stream;
  hipEvent_t e0, e1;
  WQ_HIP_CHECK(hipEventCreate(&e0));
  WQ_HIP_CHECK(hipEventCreate(&e1));
  std::vector<double> lat(cand.size(), -1.0);
  int rot = 0;
  // one call of candidate c on stream q, on the next weight copy
  auto run_cand = [&](size_t c, hipStream_t q) -> wq_status {
    const wq_weight* w = &copies[rot];
    rot = (rot + 1) % n_copies;
    return gemv ? gemv_impl(w, x, M, y, cand[c].split, cand[c].waves, cand[c].rows, ws, ws_bytes, q)
                : gemm_impl(w, x, M, y, cand[c].tile, ws, ws_bytes, q);
  };
  // Mean microseconds per call of candidate c as HIP graph replays: two rotations over
  // the copies (at least 8 calls) captured on a stream of the tuner's own, 2 replays
  // of warm-up, then replays covering about `iters` calls.  Leaves *us unchanged when
  // the graph cannot be built (the back-to-back timing then stands).
  auto time_cand_graph = [&](size_t c, double* us) -> wq_status {
    if (*us < 0) return WQ_OK;
    const int calls = std::max(8, 2 * n_copies);
    const int reps = std::max(1, iters / calls);
    hipStream_t cs = nullptr;
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
    wq_status rs = WQ_OK;
    float ms = 0.f;
    WQ_HIP_CHECK(hipStreamSynchronize(hs));
    if (hipStreamCreateWithFlags(&cs, hipStreamNonBlocking) != hipSuccess) return WQ_OK;
    if (hipStreamBeginCapture(cs, hipStreamCaptureModeRelaxed) == hipSuccess) {
      for (int i = 0; i < calls && rs == WQ_OK; ++i) rs = run_cand(c, cs);
      const hipError_t ec = hipStreamEndCapture(cs, &graph);
      if (rs == WQ_OK && ec == hipSuccess && graph &&
          hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0) == hipSuccess) {
        bool ok = hipGraphLaunch(exec, cs) == hipSuccess && hipGraphLaunch(exec, cs) == hipSuccess &&
                  hipEventRecord(e0, cs) == hipSuccess;
        for (int r = 0; ok && r < reps; ++r) ok = hipGraphLaunch(exec, cs) == hipSuccess;
        ok = ok && hipEventRecord(e1, cs) == hipSuccess && hipEventSynchronize(e1) == hipSuccess &&
             hipEventElapsedTime(&ms, e0, e1) == hipSuccess;
        if (ok) *us = (double)ms * 1000.0 / ((double)reps * calls);
        else rs = fail(WQ_ERR_HIP, "wq_tune: graph replay failed");
      }
    }
    (void)hipStreamSynchronize(cs);
    if (exec) (void)hipGraphExecDestroy(exec);
    if (graph) (void)hipGraphDestroy(graph);
    (void)hipStreamDestroy(cs);
    (void)hipGetLastError();  // a capture that could not be built leaves no sticky error
    return rs == WQ_ERR_HIP ? rs : WQ_OK;
  };
  // mean microseconds of candidate c over `iters` calls after `warmup` (negative: the
  // candidate cannot run with this workspace)
  auto time_cand = [&](size_t c, double* us) -> wq_status {
    *us = -1.0;
    if (gemv) {
      const int s = cand[c].split;
      if (s > split_units(&copies[0])) return WQ_OK;
      if (s > 1 && (!ws || ws_bytes < gemv_workspace_bytes(copies[0].N, M, s))) return WQ_OK;
    } else {
      const size_t need = gemm_workspace_bytes(copies[0].fmt, copies[0].N, M, cand[c].tile);
      if (need > 0 && (!ws || ws_bytes < need)) return WQ_OK;
      if (cand[c].tile >= kSkinnyTile0 && cand[c].tile <= kSkinnyTileLast &&
          gemm_skinny_split(cand[c].tile, M, copies[0].N) == 0)
        return WQ_OK;
      if (cand[c].tile >= kMmaTile0 && cand[c].tile <= kMmaTileLast && gemm_mma_split(cand[c].tile, M, copies[0].K) == 0)
        return WQ_OK;  // more tokens than the matrix-core GEMV kernel takes
    }
    auto run = [&]() -> wq_status { return run_cand(c, hs); };
    wq_status rs;
    for (int i = 0; i < warmup; ++i)
      if ((rs = run()) != WQ_OK) return rs;
    if (hipEventRecord(e0, hs) != hipSuccess) return fail(WQ_ERR_HIP, "hipEventRecord");
    for (int i = 0; i < iters; ++i)
      if ((rs = run()) != WQ_OK) return rs;
    if (hipEventRecord(e1, hs) != hipSuccess || hipEventSynchronize(e1) != hipSuccess)
      return fail(WQ_ERR_HIP, "hipEventSynchronize");
    float ms = 0.f;
    (void)hipEventElapsedTime(&ms, e0, e1);
    *us = (double)ms * 1000.0 / iters;
    return WQ_OK;
  };
  for (size_t c = 0; c < cand.size(); ++c)
    if ((st = time_cand(c, &lat[c])) != WQ_OK) goto out;
  {
    // Confirmation: the four fastest are timed once more, as HIP graph replays (the way
    // a decode step replays them), and that second timing decides (a single pass
    // favours whichever candidate happened to run fast).
    std::vector<size_t> order;
    for (size_t c = 0; c < cand.size(); ++c)
      if (lat[c] >= 0) order.push_back(c);
    std::stable_sort(order.begin(), order.end(), [&](size_t a, size_t b) { return lat[a] < lat[b]; });
    if (order.size() > 4) order.resize(4);
    std::sort(order.begin(), order.end());  // re-time in candidate order
    for (const size_t c : order)
      if ((st = time_cand_graph(c, &lat[c])) != WQ_OK) goto out;
  }
  {
    const int best = wq_tune_pick(lat.data(), (int)lat.size());
    if (best < 0) {
      st = fail(WQ_ERR_WORKSPACE, "wq_tune: no candidate could run");
      goto out;
    }
    if (lat_us)
      for (int i = 0; i < WQ_TUNE_LAT_SLOTS; ++i) lat_us[i] = -1.0;
    if (gemv) {
      *chosen = cand[best].split;
      if (lat_us) {
        // per split_k: the best time over the waves candidates
        for (int i = 0, s = 1; s <= kMaxSplit; s *= 2, ++i) {
          double b = -1.0;
          for (size_t c = 0; c < cand.size(); ++c)
            if (cand[c].split == s && lat[c] >= 0 && (b < 0 || lat[c] < b)) b = lat[c];
          lat_us[i] = b;
        }
      }
      st = wq_tune_cache_set("", copies[0].fmt, copies[0].K, copies[0].N, M, WQ_KIND_GEMV,
                             gemv_value(cand[best].split, cand[best].waves, cand[best].rows));
    } else {
      *chosen = cand[best].tile;
      if (lat_us)
        for (size_t c = 0; c < cand.size(); ++c)
          if (cand[c].tile >= 1 && cand[c].tile <= WQ_TUNE_LAT_SLOTS) lat_us[cand[c].tile - 1] = lat[c];
      st = wq_tune_cache_set("", copies[0].fmt, copies[0].K, copies[0].N, M, WQ_KIND_GEMM, cand[best].tile);
    }
  }
out:
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  return st;
}

wq_status wq_tune_cache_set(const char* tag, int fmt, int64_t K, int64_t N, int64_t M, int kind,
                            int value) {
  wq_status st = check_shape(fmt, K, N);
  if (st != WQ_OK) return st;
  fmt = compute_fmt(fmt);  // per-channel W4 runs (and is tuned) as group-128 W4
  if (M < 1 || (kind != WQ_KIND_GEMV && kind != WQ_KIND_GEMM))
    return fail(WQ_ERR_INVALID_ARG, "bad M or kind");
  if (kind == WQ_KIND_GEMV && !valid_gemv_value(value))
    return fail(WQ_ERR_INVALID_ARG, "GEMV value must be split_k | waves << 8 (powers of two, <= 32 / <= 16)");
  if (kind == WQ_KIND_GEMM && (value < 1 || value > WQ_GEMM_TILES))
    return fail(WQ_ERR_INVALID_ARG, "bad tile id");
  const std::string t = resolve_tag(tag);
  if (t.empty()) return fail(WQ_ERR_NO_DEVICE, "no device tag");
  std::lock_guard<std::mutex> lk(g_cache_mu);
  g_cache[Key{t, fmt, K, N, M, kind}] = value;
  return WQ_OK;
}

wq_status wq_tune_cache_get(const char* tag, int fmt, int64_t K, int64_t N, int64_t M, int kind,
                            int* value) {
  if (!value) return fail(WQ_ERR_INVALID_ARG, "value is NULL");
  const std::string t = resolve_tag(tag);
  if (t.empty()) return fail(WQ_ERR_NO_DEVICE, "no device tag");
  if (!cache_lookup(t, compute_fmt(fmt), K, N, M, kind, value)) return fail(WQ_ERR_INVALID_ARG, "no entry");
  return WQ_OK;
}

wq_status wq_tune_cache_clear(void) {
  std::lock_guard<std::mutex> lk(g_cache_mu);
  g_cache.clear();
  return WQ_OK;
}

wq_status wq_tune_cache_save(const char* path) {
  if (!path) return fail(WQ_ERR_INVALID_ARG, "path is NULL");
  FILE* f = std::fopen(path, "w");
  if (!f) return fail(WQ_ERR_CACHE_IO, std::string("cannot write ") + path);
  std::lock_guard<std::mutex> lk(g_cache_mu);
  std::fprintf(f, "# wq tuner cache v1: tag fmt K N M kind value\n");
  for (const auto& kv : g_cache)
    std::fprintf(f, "%s %d %" PRId64 " %" PRId64 " %" PRId64 " %d %d\n", kv.first.tag.c_str(),
                 kv.first.fmt, kv.first.K, kv.first.N, kv.first.M, kv.first.kind, kv.second);
  const bool ok = std::fclose(f) == 0;
  return ok ? WQ_OK : fail(WQ_ERR_CACHE_IO, std::string("cannot write ") + path);
}

wq_status wq_tune_cache_load(const char* path) {
  if (!path) return fail(WQ_ERR_INVALID_ARG, "path is NULL");
  FILE* f = std::fopen(path, "r");
  if (!f) return fail(WQ_ERR_CACHE_IO, std::string("cannot read ") + path);
  std::vector<std::pair<Key, int>> entries;
  char line[512];
  bool bad = false;
  while (std::fgets(line, sizeof line, f)) {
    if (line[0] == '#' || line[0] == '\n') continue;
    char tag[256];
    int fmt, kind, value;
    int64_t K, N, M;
    if (std::sscanf(line, "%255s %d %" SCNd64 " %" SCNd64 " %" SCNd64 " %d %d", tag, &fmt, &K, &N, &M,
                    &kind, &value) != 7 ||
        check_shape(fmt, K, N) != WQ_OK || M < 1 || (kind != WQ_KIND_GEMV && kind != WQ_KIND_GEMM) ||
        (kind == WQ_KIND_GEMV && !valid_gemv_value(value)) ||
        (kind == WQ_KIND_GEMM && (value < 1 || value > WQ_GEMM_TILES))) {
      bad = true;
      break;
    }
    entries.push_back({Key{tag, fmt, K, N, M, kind}, value});
  }
  std::fclose(f);
  if (bad) return fail(WQ_ERR_CACHE_IO, std::string("malformed tuner cache ") + path);
  std::lock_guard<std::mutex> lk(g_cache_mu);
  for (auto& e : entries) g_cache[e.first] = e.second;
  return WQ_OK;
}

}  // extern "C"
