// Internal declarations shared by the library's translation units (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "../../include/wq.h"

namespace wq {

constexpr int kGroup = 128;        // group size along K for the group-128 formats
constexpr int kMaxSplit = 32;      // largest split_k of the tuning grid
constexpr int kGemvMaxM = 7;       // tokens < 8 take the GEMV
constexpr int kMmaTokens = 16;     // tokens the matrix-core GEMV kernel takes (the GEMM's few-token tiles)
constexpr int kGemvTileRows = 16;    // output rows per GEMV workgroup tile (and per
                                     // gfx950 metadata tile of the group-128 formats)
constexpr int kGemvMaxWaves = 16;    // waves per GEMV workgroup (intra-workgroup K split)
constexpr int kGemvPrefetch = WQ_GEMV_PREFETCH;  // "rows" flag: slice prefetch
constexpr int kGemvMfma = WQ_GEMV_MFMA;          // "rows" flag: matrix-core GEMV

// Thread-local error text behind wq_last_error().
void set_error(const std::string& msg);
wq_status fail(wq_status st, const std::string& msg);
wq_status hip_fail(hipError_t e, const char* what);

#define WQ_HIP_CHECK(call)                                   \
  do {                                                       \
    hipError_t e_ = (call);                                  \
    if (e_ != hipSuccess) return ::wq::hip_fail(e_, #call);  \
  } while (0)

// uint4 formats (grouped and per output channel)
inline bool is_w4(int fmt) {
  return fmt == WQ_FMT_W4_G128 || fmt == WQ_FMT_W4_PC || fmt == WQ_FMT_W4_G32 || fmt == WQ_FMT_W4_G64;
}
// k per group of a format's gfx950 metadata (what the compute kernels fold by): 0 for
// per-channel W8; per-channel W4 is laid out as group-128 (see compute_view)
inline int meta_group(int fmt) {
  switch (fmt) {
    case WQ_FMT_W8_G32: case WQ_FMT_W4_G32: return 32;
    case WQ_FMT_W8_G64: case WQ_FMT_W4_G64: return 64;
    case WQ_FMT_W8_PC: return 0;
    default: return kGroup;
  }
}
// groups of 32 or 64 (the kernels that take them run one template per group size)
inline bool small_group(int fmt) { const int g = meta_group(fmt); return g == 32 || g == 64; }
// kernel family of a format: the group-128 kernels (templated on the group size where
// they take groups of 32 and 64) serve every grouped format of their code width
inline int family(int fmt) {
  if (fmt == WQ_FMT_W8_PC) return WQ_FMT_W8_PC;
  return is_w4(fmt) ? WQ_FMT_W4_G128 : WQ_FMT_W8_G128;
}
// The compute kernels take per-channel W4 in the gfx950 layout as group-128 W4: that
// layout repeats each row's scale and zero-point in every 128-k group.
inline int compute_fmt(int fmt) { return fmt == WQ_FMT_W4_PC ? WQ_FMT_W4_G128 : fmt; }
inline wq_weight compute_view(const wq_weight& w) {
  wq_weight v = w;
  v.fmt = (decltype(v.fmt))compute_fmt(v.fmt);
  return v;
}

// Shape/format validation shared by every entry point (no device access).
wq_status check_shape(int fmt, int64_t K, int64_t N);
wq_status check_weight(const wq_weight* w, int want_layout);

// Number of 16-row tiles of N (the gfx950 metadata of group-128 formats is padded to them).
__host__ __device__ inline int64_t row_tiles(int64_t N) { return (N + kGemvTileRows - 1) / kGemvTileRows; }

// gfx950 code layout: byte b of packed row n (row_bytes = K for int8, K/2 for uint4)
// lives in the 1 KB slice b / 1024 of its 16-row tile; a tile stores its slices one
// after another and a slice stores its rows one after another, so the 16 rows x
// 1 KB a GEMV wave reads for one slice are one contiguous block.
constexpr int kSliceBytes = 1024;
__host__ __device__ inline size_t tiled_offset(int64_t n, int64_t b, int64_t N, int64_t row_bytes) {
  const int64_t t = n / kGemvTileRows, r = n % kGemvTileRows;
  const int64_t nr = N - t * kGemvTileRows < kGemvTileRows ? N - t * kGemvTileRows : kGemvTileRows;
  const int64_t sl = b / kSliceBytes, j = b % kSliceBytes;
  const int64_t w = row_bytes - sl * kSliceBytes < kSliceBytes ? row_bytes - sl * kSliceBytes : kSliceBytes;
  return (size_t)(t * kGemvTileRows * row_bytes + nr * kSliceBytes * sl + r * w + j);
}

// Streaming 16-byte load with the non-temporal hint: weights are read once per call,
// and loads marked so stream from HBM about 8-10 % faster on MI355X (measured with a
// plain read kernel) than loads that allocate in the caches like x does.
__device__ __forceinline__ uint4 load_stream16(const void* p) {
  const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
  uint4 v;
  v.x = __builtin_nontemporal_load(q + 0);
  v.y = __builtin_nontemporal_load(q + 1);
  v.z = __builtin_nontemporal_load(q + 2);
  v.w = __builtin_nontemporal_load(q + 3);
  return v;
}

// --- kernel launchers (implemented in the .hip files) ---
wq_status launch_pack(const float* w, const wq_weight* out, hipStream_t s);
wq_status launch_pack_bf16(const uint16_t* w, const wq_weight* out, hipStream_t s);
// x'[m][j] = x[m][perm[j]] for m < M, j < K (K % 8 == 0, xp 16-byte aligned); an
// index outside [0, K) reads as +0.
wq_status launch_perm_gather(const uint16_t* x, const int32_t* perm, uint16_t* xp, int64_t M, int64_t K,
                             hipStream_t s);
wq_status launch_repack(const wq_weight* src, const wq_weight* dst, bool to_gfx950, hipStream_t s);
// xf: fp16 activations (x and y in fp16; the dot2 launch options without prefetch)
// res: NULL, or a residual of y's type and shape added to the fp32 result before the one
// rounding of y (it may be y itself)
wq_status launch_gemv(const wq_weight* w, const uint16_t* x, int M, uint16_t* y, int split_k,
                      int waves, int rows, void* ws, hipStream_t s, bool xf = false,
                      const uint16_t* res = nullptr);
// Rows per GEMV wave (4, 8 or 16) and waves per workgroup when none is tuned or given.
int gemv_default_rows(int64_t K, int64_t N, int fmt, int M);
int gemv_default_waves(int64_t K, int64_t N, int fmt, int M, int split_k, int rows);
// Largest waves per GEMV workgroup that fits the registers at this format, M and
// rows per wave (4, 8 or 16, optionally | kGemvPrefetch; 16, 32 or 64 |
// kGemvMfma); 0 for any other rows value and for a flag where it is not offered.
int gemv_max_waves(int fmt, int M, int rows);
// K slices of the GEMV (64 lanes x one 16-byte chunk: 1024 k int8, 2048 k uint4);
// split-K ranges are whole slices.
int64_t gemv_slices(int64_t K, int fmt);
// GEMM tiles kSkinnyTile0 .. WQ_GEMM_TILES are the skinny kernel (M <= kSkinnyMaxM)
// with split-K 2, 4, 8, 16, capped so that split * M <= kSkinnyMaxSplitTokens and the
// grid stays within twice kSkinnyMaxBlocks workgroups (split 1 when the caller gives
// no workspace).
constexpr int kSkinnyTile0 = 5, kSkinnyTileLast = 8;
constexpr int kSkinnyMaxM = 128;
constexpr int kSkinnyMaxSplitTokens = 1024;
constexpr int kSkinnyMaxBlocks = 1024;
int gemm_skinny_split(int tile, int64_t M, int64_t N);  // 0 when the tile is not a skinny one
// GEMM tiles kDmaSplitTile0 .. kDmaSplitTileLast are the 8-wave LDS-DMA tile with split-K
// 2, 4, 8 over K steps (whole groups for group-128), capped so that the grid stays
// within two workgroups per CU and the fp32 partials within kDmaSplitMaxBytes.
constexpr int kDmaSplitTile0 = 10, kDmaSplitTileLast = 12;
// GEMM tile kDmaSplit3Tile: the same with split-K 3 (a single partial round of 128 ..
// 170 tiles on 256 CUs becomes 1.5 .. 2 rounds of thirds instead of 2 .. 2.7 of halves).
constexpr int kDmaSplit3Tile = 24;
constexpr int64_t kDmaSplitMaxBytes = int64_t(256) << 20;
int gemm_dma_split(int fmt, int tile, int64_t M, int64_t N);  // 0 when the tile is not a split one
// GEMM tile kDmaTailTile is tile 9 with the tiles of a partial last round (fewer than
// half the CUs' worth) split over K into up to kDmaTailMaxSplit ranges, so that round
// spreads over the idle CUs; gemm_dma_tail returns that split (1: nothing to split)
// and sets *tail0 to the number of tiles that stay whole.
constexpr int kDmaTailTile = 13, kDmaTailMaxSplit = 4;
// GEMM tiles kDma64Tile0 .. kDma64TileLast: the LDS-DMA pipeline with 64-row x tiles
// (a few tokens: the weights stream as in tile 9 with a quarter of its x traffic and
// MFMA work) and split-K 1, 2, 4, capped as the split LDS-DMA tiles.
constexpr int kDma64Tile0 = 14, kDma64TileLast = 16;
// GEMM tiles kDma64DeepTile0 .. kDma64DeepTileLast: the same 64-row tiles with split-K 8
// and 16, for narrow N (N = 5120 has 20 column tiles of 256: split 4 keeps 80
// workgroups on 256 CUs, each holding only its own few DMA stages in flight).
constexpr int kDma64DeepTile0 = 25, kDma64DeepTileLast = 26;
// GEMM tiles kDma128DeepTile0 .. kDma128DeepTileLast: the 128-row tiles with split-K 8 and
// 16 (narrow N at 129..256 tokens: N = 5120 has 20 column tiles).
constexpr int kDma128DeepTile0 = 27, kDma128DeepTileLast = 28;
// GEMM tiles kDma128Tile0 .. kDma128TileLast: the same with 128-row x tiles (mid M on
// narrow N, where 256-row tiles leave most CUs idle), split-K 1, 2, 4.
constexpr int kDma128Tile0 = 17, kDma128TileLast = 19;
// GEMM tiles kMmaTile0 .. kMmaTileLast: the matrix-core GEMV kernel for 8 ..
// kMmaTokens tokens (its A operand holds 16 tokens, so it streams the weights as at one
// token): 16 NB output rows per workgroup with NB = 1, 2, 4 (tiles 20, 21, 22) and NB = 1
// with split-K 2 (tile 23; fp32 partials in the workspace, split 1 without room for
// them).  More tokens take tile 14 (tile 2 when K % 64 != 0).
constexpr int kMmaTile0 = 20, kMmaTileLast = 23;
// split-K of a tile kMmaTile0 .. kMmaTileLast at M tokens (0: not such a tile, or M too large)
int gemm_mma_split(int tile, int64_t M, int64_t K);
// The tile that runs for groups of 32 or 64: their kernels are tile 2's and the LDS-DMA
// tiles' (9..19, 24..28); tiles 1, 3 and 4 run as tile 9, the skinny and matrix-core GEMV
// tiles (5..8, 20..23) as tile 14.
inline int small_group_tile(int tile) {
  if (tile == 1 || tile == 3 || tile == 4) return 9;
  if ((tile >= kSkinnyTile0 && tile <= kSkinnyTileLast) || (tile >= kMmaTile0 && tile <= kMmaTileLast))
    return kDma64Tile0;
  return tile;
}
// rows per x tile of the row-tiled LDS-DMA tiles 14..19, 25..28 (0 for other tiles)
inline int gemm_dma_rows(int tile) {
  if ((tile >= kDma64Tile0 && tile <= kDma64TileLast) || (tile >= kDma64DeepTile0 && tile <= kDma64DeepTileLast))
    return 64;
  if ((tile >= kDma128Tile0 && tile <= kDma128TileLast) || (tile >= kDma128DeepTile0 && tile <= kDma128DeepTileLast))
    return 128;
  return 0;
}
// rows per x tile of the LDS-DMA tiles 3, 4 and 9..13: 256 for per-channel W8; 128 for
// the group-128 formats, whose exact kernel keeps a second accumulator set (each group's
// partial sums, added into the first times the group scale) that a 256-row tile has no
// registers for
inline int gemm_big_dma_rows(int fmt) { return fmt == WQ_FMT_W8_PC ? 256 : 128; }
int gemm_dma64_split(int tile, int64_t M, int64_t N);  // 0 when the tile is not one of 14..19, 25..28
int gemm_dma_tail(int fmt, int64_t M, int64_t N, int* tail0);
// Compute units of the current device (kDefaultCUs, MI355X's count, if it cannot be queried).
constexpr int kDefaultCUs = 256;
int device_cus();
// Workspace bytes a GEMM tile needs at this M (fp32 split-K partials; 0 for most tiles).
size_t gemm_workspace_bytes(int fmt, int64_t N, int64_t M, int tile);
// Bytes with which a tile takes its fastest path: for the group-128 LDS-DMA tiles
// (9..19, 24..28) also x converted to fp16 once per call (M x K x 2 bytes after the partials,
// at a 256-byte boundary); without that room the tile converts x in LDS.
size_t gemm_workspace_full_bytes(int fmt, int64_t K, int64_t N, int64_t M, int tile);
// xf: fp16 activations (x and y in fp16): tile 2's kernel, and for the grouped formats the
// LDS-DMA tiles, which read the fp16 x as their operand (act_tile gives what runs)
wq_status launch_gemm(const wq_weight* w, const uint16_t* x, int64_t M, uint16_t* y, int tile,
                      void* ws, size_t ws_bytes, hipStream_t s, bool xf = false, const uint16_t* res = nullptr);
// the GEMM tile that runs for fp16 activations: the LDS-DMA tiles have fp16 forms (tiles 3
// and 4 run as 9); the skinny and matrix-core GEMV tiles run as tile 14, tile 1 as tile 2's
// kernel; the grouped formats map as small_group_tile does
inline int act_tile(int fmt, int tile) {
  if (fmt != WQ_FMT_W8_PC) return small_group_tile(tile);
  if (tile == 3 || tile == 4) return 9;
  if ((tile >= kSkinnyTile0 && tile <= kSkinnyTileLast) || (tile >= kMmaTile0 && tile <= kMmaTileLast))
    return kDma64Tile0;
  return tile == 1 ? 2 : tile;
}

// Workspace bytes for a GEMV with the given split (fp32 partials of every slice).
size_t gemv_workspace_bytes(int64_t N, int64_t M, int split_k);

// LM head + top-k: chunks of 2048 logits per workgroup of the first kernel; the merge
// kernel sorts up to kTopkMergeMax chunk candidates of a row in LDS.
constexpr int kTopkMaxK = 64;
constexpr int kTopkMergeMax = 8192;
int topk_chunks(int64_t V);
wq_status launch_topk(const uint16_t* logits, int64_t M, int64_t V, int k, float temperature, const float* u,
                      uint64_t* cand, uint16_t* top_vals, int32_t* top_idx, int32_t* tokens, hipStream_t s);

// Grouped (mixture-of-experts) layer: E experts stacked with the given byte strides.
wq_status launch_moe(const wq_weight* w, int E, const uint16_t* x, const int32_t* offsets, int64_t T, uint16_t* y,
                     bool gated, size_t qw_stride, size_t sc_stride, size_t zs_stride, hipStream_t s);

// Device tag "<arch>:<CUs>" of the current device; empty on failure.
std::string current_device_tag();

}  // namespace wq
