/*
 * wq.h -- C ABI of the weight-only quantized linear library for MI355X (gfx950).
 *
 * The layer computes y = x . dequant(Wq, s[, z])^T with bf16 activations x[M][K],
 * quantized weights W[N][K] (N output channels, K input features), fp32
 * accumulation and bf16 output y[M][N].  This is the int8 weight-only linear of
 * the tileInfer README (feature table, "INT8 Weight-Only Quantization": int8
 * weights with one scale per output channel, bf16 activations; "Key
 * Optimizations": decode dequantizes in registers inside a GEMV, prefill
 * dequantizes to bf16 on the fly for a GEMM), extended to the group-128 INT8 and
 * INT4 formats of "Marlin register and launch scheduling benchmark" ("Validation
 * and limits"; "Full inference" for the group-128 vocabulary heads).
 *
 * Conventions shared by every entry point:
 *   - Pointers named in a wq_weight, x, y and ws are DEVICE pointers (memory from
 *     hipMalloc or a PyTorch HIP tensor); size_t/int64_t out-parameters and the
 *     path strings are HOST pointers.
 *   - The caller owns every buffer.  The library never allocates device memory
 *     (its only device memory of its own is the static scratch of wq_linear_static,
 *     which comes with the loaded code), never frees anything it was given and keeps
 *     no pointer after a call returns.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Device work is
 *     enqueued asynchronously on it; wq_gemv, wq_gemm and wq_linear neither
 *     synchronize nor read device memory on the host, so they may be captured
 *     into a HIP graph.  Only wq_tune synchronizes.
 *   - Every precondition is checked on the host before anything is enqueued; on
 *     an error status nothing has been written.  A failed HIP call returns
 *     WQ_ERR_HIP.  wq_last_error() gives the detail text (per calling thread).
 *   - bf16 and fp16 values are passed as their 16-bit patterns (uint16_t).
 */
#ifndef WQ_H
#define WQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define WQ_ABI_VERSION 1

typedef enum {
  WQ_OK = 0,
  WQ_ERR_INVALID_ARG = 1,  /* null pointer, bad size or value                       */
  WQ_ERR_UNSUPPORTED = 2,  /* format/layout/shape combination not provided          */
  WQ_ERR_ALIGNMENT = 3,    /* a device pointer is not 16-byte aligned               */
  WQ_ERR_WORKSPACE = 4,    /* workspace missing or smaller than wq_workspace_size   */
  WQ_ERR_NO_DEVICE = 5,    /* no HIP device is visible                              */
  WQ_ERR_HIP = 6,          /* a HIP runtime call or kernel launch failed            */
  WQ_ERR_CACHE_IO = 7      /* tuner cache file could not be read or written         */
} wq_status;

/* Weight formats (the quantization recipe is stated at wq_pack). */
typedef enum {
  WQ_FMT_W8_PC = 0,    /* int8, symmetric, one bf16 scale per output channel       */
  WQ_FMT_W8_G128 = 1,  /* int8, symmetric, one bf16 scale per 128 consecutive k     */
  WQ_FMT_W4_G128 = 2,  /* uint4, asymmetric, fp16 scale + uint4 zero per 128 k      */
  WQ_FMT_W4_PC = 3,    /* uint4, asymmetric, fp16 scale + uint4 zero per channel    */
  WQ_FMT_W8_G32 = 4,   /* int8 as W8_G128 with one bf16 scale per 32 consecutive k  */
  WQ_FMT_W8_G64 = 5,   /* int8 as W8_G128 with one bf16 scale per 64 consecutive k  */
  WQ_FMT_W4_G32 = 6,   /* uint4 as W4_G128 with a scale and zero per 32 k           */
  WQ_FMT_W4_G64 = 7    /* uint4 as W4_G128 with a scale and zero per 64 k           */
} wq_format;
/* The grouped formats (W8_G32/G64/G128, W4_G32/G64/G128; Gs = 32, 64 or 128 k per
 * group, G = K / Gs groups per row) share one layout, written below for Gs = 128.
 * Every grouped and W4 format needs K % 128 == 0 (the kernels' K steps); W4 needs
 * N % 8 == 0.  The Marlin page's "Validation and limits" lists per-channel scales and
 * groups of 32, 64 and 128 for INT4 and INT8 weights. */

/* Memory layouts of a packed weight.
 *
 * WQ_LAYOUT_CANONICAL (interchange; what wq_pack writes):
 *   W8:  qweight int8 [N][K] row-major; scales bf16 [N] (per channel) or [N][G].
 *   W4:  qweight uint32 [N][K/8], bits 4j..4j+3 of word (n,c) hold q[n][8c+j];
 *        scales fp16 [N][G];
 *        zeros uint32 [G][N/8], bits 4j..4j+3 of word (g,c) hold z[8c+j][g].
 *   W4 per channel: as W4 with one group: scales fp16 [N]; zeros uint32 [N/8].
 *
 * WQ_LAYOUT_GFX950 (what the compute kernels read; written by wq_repack).  N16 =
 * ceil(N/16) tiles of 16 output rows; metadata entries for rows >= N are 0.
 *   Codes (both formats) keep the bytes of each packed row (row_bytes = K for int8,
 *   K/2 for uint4) but store them tile by tile and, inside a tile, 1 KB slice by
 *   slice: byte b of row n = 16t + r (tile t holding nr = min(16, N - 16t) rows)
 *   lies in slice sl = b / 1024 of width w = min(1024, row_bytes - 1024 sl) at
 *       16 * row_bytes * t + nr * 1024 * sl + r * w + (b mod 1024),
 *   so the 16 rows x 1 KB that a GEMV wave reads for one K slice are contiguous.
 *   W8:  the code bytes hold u = q + 128 (the sign bit of q flipped), so that a
 *        byte placed under the fp16 exponent byte 0x64 reads 1024 + u exactly;
 *        scales bf16 [N] for per-channel; for the grouped formats bf16 [N16][G][16]
 *        with element (t,g,j) = s[16t+j][g]: the 16 rows of a tile side by side.
 *   W4:  each 32-bit word of codes holds the same 8 codes as the canonical word with
 *        the nibbles interleaved: bits 4p..4p+3 hold q[n][8c + (2p mod 8) + (p >= 4)],
 *        i.e. nibble order q0 q2 q4 q6 q1 q3 q5 q7, so that (word >> 4i) & 0x000F000F
 *        yields the consecutive pair (q[8c+2i], q[8c+2i+1]) in the two 16-bit halves;
 *        scales fp16 [N16][G][16] as for grouped W8;
 *        zeros uint8 [N16][G][8], byte (t,g,h) holds z[16t+2h][g] in bits 0..3 and
 *        z[16t+2h+1][g] in bits 4..7.
 *   W4 per channel: exactly the W4 group-128 layout (same sizes) with each row's one
 *        scale and zero-point written into every one of its K/128 groups, so that the
 *        group-128 kernels compute it unchanged (the group scales multiply equal
 *        factors: the same products in another fp32 summation order); wq_unrepack
 *        reads the first group back.
 */
typedef enum { WQ_LAYOUT_CANONICAL = 0, WQ_LAYOUT_GFX950 = 1 } wq_layout;

/* Non-owning view of one packed weight.  zeros is NULL for the W8 formats. */
typedef struct {
  int32_t fmt;     /* wq_format */
  int32_t layout;  /* wq_layout */
  int64_t K;       /* input features (reduction length)  */
  int64_t N;       /* output channels                     */
  void* qweight;
  void* scales;
  void* zeros;
} wq_weight;

/* Which kernel family wq_linear uses for M tokens. */
typedef enum { WQ_KIND_GEMV = 0, WQ_KIND_GEMM = 1 } wq_kind;

/* ---------------------------------------------------------------- host info */

/* WQ_ABI_VERSION of the built library. */
int wq_abi_version(void);

/* Static English text for a status code (never NULL). */
const char* wq_status_string(int status);

/* Detail text of the last failing call on this thread ("" if none). */
const char* wq_last_error(void);

/* Bytes of qweight, scales and zeros for a format/layout/shape (host only, no
 * device access).  Shape rules: K > 0, N > 0, K % 16 == 0; the grouped formats and W4
 * per channel need K % 128 == 0; W4 needs N % 8 == 0.  zero_bytes is 0 for W8.  Any out-pointer
 * may be NULL. */
wq_status wq_packed_sizes(int fmt, int layout, int64_t K, int64_t N, size_t* qweight_bytes,
                          size_t* scale_bytes, size_t* zero_bytes);

/* Kernel family for M tokens: M < 8 -> WQ_KIND_GEMV, M >= 8 -> WQ_KIND_GEMM.  The
 * threshold and the token count M = numel(x) / K follow "Heuristic: Mit han lab Llm
 * awq Kernel Selection Thresholds" ("The Insight (Rule of Thumb)", Linear Kernel,
 * and its awq/quantize/qmodule.py excerpt).  Returns -1 for M < 1. */
int wq_dispatch_kind(int64_t M);

/* --------------------------------------------------------------- packing */

/* Quantize an fp32 weight w[N][K] (device, row-major) into `out`, which must
 * describe CANONICAL-layout buffers of wq_packed_sizes bytes.  Recipe (IEEE fp32,
 * round to nearest even, correctly rounded division):
 *   W8 (group G = K for per-channel, else the format's 32, 64 or 128):
 *     a = max|w| over the group; s = bf16(a / 127);
 *     q = 0 if s == 0 else clamp(rint(w / s), -127, 127)   (divides by the stored s)
 *   W4 (groups of 32, 64 or 128, or one group per output channel for WQ_FMT_W4_PC:
 *   the INT4 cases of the Marlin page's "Validation and limits"):
 *     hi = max w, lo = min w over the group; s = fp16((hi - lo) / 15);
 *     s == 0 -> z = 0, q = 0; else z = clamp(rint(-lo / s), 0, 15),
 *     q = clamp(rint(w / s) + z, 0, 15).
 * The output is bit-exact and deterministic.  `w` must not alias the outputs. */
wq_status wq_pack(const float* w, const wq_weight* out, void* stream);

/* wq_pack for a bf16 weight w[N][K] (device, row-major, 8-byte aligned): each value
 * widens exactly to fp32 and the recipe above runs on the widened weight, so the
 * output is bit-identical to wq_pack of that fp32 copy (checkpoints stored in bf16
 * need no fp32 staging buffer). */
wq_status wq_pack_bf16(const void* w, const wq_weight* out, void* stream);

/* CANONICAL -> GFX950 (wq_repack) and back (wq_unrepack); src and dst describe
 * distinct buffers of the same format and shape in the named layouts.  The two are
 * exact inverses on every valid packed weight. */
wq_status wq_repack(const wq_weight* src, const wq_weight* dst, void* stream);
wq_status wq_unrepack(const wq_weight* src, const wq_weight* dst, void* stream);

/* ------------------------------------------------------------- the linear */

/* Workspace bytes needed by wq_gemv / wq_gemm / wq_linear for this weight and M
 * under any split the library may pick (host only): fp32 partial sums of the
 * ranges of a cross-workgroup K split -- 32 * M * N * 4 bytes for M < 8 (GEMV); for
 * M >= 8 the largest split * M * N * 4 of the split GEMM tiles: the skinny tiles (M <=
 * 128; split <= 16, split * M <= 1024, at most 2048 workgroups) and the split-K
 * LDS-DMA tiles (split <= 16, at most 512 workgroups, at most 256 MiB) -- or the
 * partials of tile 13's split last round (sized for the current device's CU count, 256
 * when none is visible); 0 when no split applies.  For the group-128 formats the
 * LDS-DMA tiles 9..19, 24..28 also use M * K * 2 bytes after the partials (at a 256-byte
 * boundary) for x converted to fp16 once per call (each row scaled by a power of two
 * so that it converts exactly), then M * 4 bytes (at a 256-byte boundary) for the row
 * scales; given less, they convert x inside every workgroup instead, unscaled (same
 * results; slower, and much slower where x holds values fp16 cannot hold exactly, such
 * as magnitudes below 2^-17), so that part is never required.
 * The contents are scratch: no initialisation is needed and nothing is kept between
 * calls.  Calls that share a workspace must not run concurrently. */
wq_status wq_workspace_size(const wq_weight* w, int64_t M, size_t* bytes);

/* Decode GEMV, 1 <= M <= 7 (the "Key Optimizations" register-dequant GEMV of the
 * tileInfer README).  w must be in the GFX950 layout.  x: bf16 [M][K], y: bf16
 * [M][N], row-major; x 16-byte aligned.
 *
 * K is split at two levels.  Inside a workgroup, 1..16 waves share a tile of output
 * rows and interleave over its K range; their fp32 partial sums are added in LDS in
 * wave order.  Across workgroups, split_k slices (the split_k of "Heuristic: Mit han
 * lab Llm awq Kernel Selection Thresholds": K partitioned across thread blocks)
 * each write fp32 partials to the workspace (the FP32 reduction scratch of the
 * Marlin page's intro) and a second kernel adds them in range order.  K is cut into
 * slices of 1024 (int8) or 2048 (uint4) k, each a run of whole 128-groups; a split
 * range is a run of whole slices.  Results are bit-identical from run to run for a
 * given (split_k, waves).
 *
 * split_k: 0 = the tuned (split_k, waves) of this shape (1 slice with the default
 * waves when untuned, or when the tuned split needs more workspace than given),
 * else a power of two in 1..wq_gemv_max_split(fmt, K); waves then take the default
 * for the shape.  ws/ws_bytes may be NULL/0 when split_k resolves to 1. */
wq_status wq_gemv(const wq_weight* w, const void* x, int64_t M, void* y, int split_k, void* ws,
                  size_t ws_bytes, void* stream);

/* Largest split_k the GEMV accepts for a format and K (host only): split-K ranges
 * are whole K slices of 1024 (int8) or 2048 (uint4) k, so this is the largest power
 * of two <= min(32, number of slices).  -1 for an invalid format or K. */
int wq_gemv_max_split(int fmt, int64_t K);

/* rows flag of wq_gemv_ex / wq_gemv_max_waves: each wave loads its next K slice while
 * it multiplies the current one (a second register set; offered where that set is
 * small: 4 * rows + M * (8 for int8, 16 for uint4) <= 48). */
#define WQ_GEMV_PREFETCH 0x100

/* rows flag of wq_gemv_ex / wq_gemv_max_waves: the matrix-core GEMV.  rows = 16 * NB |
 * WQ_GEMV_MFMA with NB in {1, 2, 4} 16-row tiles per workgroup; its 1..8 waves
 * interleave over 128-k units of the workgroup's K range and multiply on
 * v_mfma_f32_16x16x32 (bf16 and fp16) with exact code values, so its cost barely
 * grows with M; the fp32 partial sums meet in LDS in wave order.  Offered for the
 * per-channel and group-128 formats (a 16x16x32 instruction sums k of four 32-k
 * blocks, which groups of 32 or 64 would scale differently). */
#define WQ_GEMV_MFMA 0x200

/* Largest waves per GEMV workgroup for a format, 1 <= M <= 7 and rows per wave (4, 8
 * or 16, optionally | WQ_GEMV_PREFETCH; or 16, 32, 64 | WQ_GEMV_MFMA) (host
 * only): the register budget per lane shrinks as a workgroup grows, so larger M and
 * more rows allow fewer waves.  -1 for an invalid argument or a flag that is not
 * offered at this format, M and rows. */
int wq_gemv_max_waves(int fmt, int64_t M, int rows);

/* wq_gemv with the work decomposition explicit: split_k >= 1 as above; rows: output
 * rows per wave, 4, 8 or 16, optionally | WQ_GEMV_PREFETCH, or the matrix-core GEMV
 * (16, 32 or 64 | WQ_GEMV_MFMA) (0 = the default for the shape; a flag that is
 * not offered: WQ_ERR_UNSUPPORTED); waves per workgroup: 0
 * (the default: one K slice per wave, as many as the registers allow) or
 * 1..wq_gemv_max_waves(fmt, M, rows) (else WQ_ERR_UNSUPPORTED).  For tests and
 * tuning. */
wq_status wq_gemv_ex(const wq_weight* w, const void* x, int64_t M, void* y, int split_k, int waves,
                     int rows, void* ws, size_t ws_bytes, void* stream);

/* Prefill GEMM, M >= 1 (used by wq_linear for M >= 8; smaller M are accepted so
 * the two paths can be compared), the tileInfer README's dequantize-to-bf16 GEMM
 * ("Key Optimizations"): every tile multiplies exact code values (q, or q - z) by x on
 * the matrix cores with fp32 accumulation; the per-channel scale is applied to the
 * finished fp32 sum, group scales to each group's fp32 partial sum, so an output carries
 * only fp32 summation and the final bf16 rounding.  The group-128 LDS-DMA tiles (9..19, 24..28)
 * multiply fp16 code values by fp16 copies of x: with the workspace's room for x (see
 * wq_workspace_size) each row is scaled by a power of two so that it converts exactly;
 * a workgroup whose x fp16 still cannot hold exactly recomputes its tile with bf16 codes
 * against bf16 x.  w must be in the GFX950 layout; x: bf16 [M][K], y: bf16 [M][N].
 *
 * tile: 0 = the tuned tile (a default by M and format when untuned), else
 *   1  256 x 256 workgroup tile (256 x 128 for group-128), 4 waves, LDS-staged;
 *   2  128 x 128 tile, 4 waves of 64 x 64;
 *   3  per-channel W8, K % 64 == 0: 256 x 256 tile fed by LDS-DMA, 2 x 2 waves;
 *   4  as 3 with 1 x 4 waves;
 *   9  as 3 with 8 waves (2 x 4, two per SIMD); for group-128 the LDS-DMA tile with
 *      fp16 code values and a 128 x 256 workgroup tile (eight waves of 128 x 32: the
 *      group partial sums need a second accumulator set) (tiles 3 and 4 for group-128,
 *      and 3, 4, 9-13 for other shapes: tile 1);
 *   10..12  tile 9 with split-K 2, 4, 8 (ranges of whole groups for group-128; fp32
 *      partials in the workspace, added in range order), capped so that the grid
 *      stays within 512 workgroups and the partials within 256 MiB (needs that
 *      workspace, else WQ_ERR_WORKSPACE; with tile 0 and too small a workspace the
 *      split drops to 1);
 *   13  tile 9 with the tiles of a partial last round split over K: when the tile
 *      count exceeds the CU count C by r <= C/2 (864 = 3 x 256 + 96 at M = 2048, N =
 *      27648 for per-channel W8), the last r tiles run as min(4, C / r) K ranges each,
 *      writing an fp32 block of the tile's size per range to the workspace (r x ranges x
 *      256 KiB, 128 KiB for group-128; needs it, else WQ_ERR_WORKSPACE; with tile 0 and
 *      too small a workspace it runs as tile 9), and a second kernel adds them in range
 *      order; other shapes: tile 9;
 *   14..16  K % 64 == 0: the LDS-DMA pipeline of tile 9 with 64-row x tiles (1 x 8
 *      waves; group-128 as tile 9), split-K 1, 2, 4 (partials as for 10..12, capped
 *      so that the grid stays within 512 workgroups; 15 and 16 need that workspace,
 *      else WQ_ERR_WORKSPACE); the default for 17..128 tokens; other shapes: tile 1;
 *   17..19  as 14..16 with 128-row x tiles (mid M on narrow N, where the 256-row
 *      tiles leave most compute units idle), split-K 1, 2, 4; 18 and 19 need the
 *      workspace; the default for 129..256 tokens; other shapes: tile 1;
 *   5..8  M <= 128, K % 128 == 0: the skinny kernel with split-K 2, 4, 8, 16 (capped
 *      as in wq_workspace_size; needs that workspace, else WQ_ERR_WORKSPACE; with
 *      tile 0 and too small a workspace the split drops to 1); other shapes: tile 2;
 *   20..22  M <= 16: the matrix-core GEMV (WQ_GEMV_MFMA) with 16, 32 or 64 rows per
 *      workgroup: its A operand holds 16 tokens, so 8..16 tokens stream the weights
 *      at about the cost of one; 23: as 20 with split-K 2 (needs 2 * M * N * 4 bytes
 *      of workspace, else WQ_ERR_WORKSPACE; with tile 0 and too small a workspace the
 *      split drops to 1); M > 16: tile 14 (tile 2 when K % 64 != 0);
 *   24  tile 9 with split-K 3 (capped and needing the workspace as 10..12): a single
 *      partial round of tiles (160 per-channel tiles at M = 2048, N = 5120) becomes
 *      work for more of the CUs;
 *   25, 26  as 14..16 with split-K 8 and 16 (capped and needing the workspace as
 *      15 and 16): narrow N at a few tokens (N = 5120 has 20 column tiles) spread over
 *      more of the CUs; the default for 17..128 tokens where splits 1..4 leave fewer
 *      than 200 workgroups; other shapes: tile 1;
 *   27, 28  as 17..19 with split-K 8 and 16 (capped and needing the workspace as 18
 *      and 19): narrow N at 129..256 tokens; other shapes: tile 1.
 * Groups of 32 and 64 run tiles 2 and 9..19, 24..28 as described for group-128 (their
 * kernels fold every group's partial sum in as a group-128 tile does); tiles 1, 3 and
 * 4 run as tile 9, tiles 5..8 and 20..23 as tile 14. 
 * ws/ws_bytes may be NULL/0 for tiles 1-4 and 9.  Results are bit-identical from run
 * to run for a given tile, device and workspace size. */
#define WQ_GEMM_TILES 28
wq_status wq_gemm(const wq_weight* w, const void* x, int64_t M, void* y, int tile, void* ws,
                  size_t ws_bytes, void* stream);

/* The layer: M = tokens; M < 8 -> wq_gemv with the tuned split_k, else wq_gemm with
 * the tuned tile (see wq_dispatch_kind). */
wq_status wq_linear(const wq_weight* w, const void* x, int64_t M, void* y, void* ws,
                    size_t ws_bytes, void* stream);

/* ----------------------------------------------- fp16 activations */

/* Activation types of the *_act entry points: the 16-bit type of x and of y. */
#define WQ_ACT_BF16 0
#define WQ_ACT_F16 1

/* The layer, the GEMV and the GEMM with x and y in the given activation type: the FP16
 * and BF16 activations that the Marlin page's "Validation and limits" lists, over the
 * same weight formats.  WQ_ACT_BF16 is wq_linear / wq_gemv_ex / wq_gemm.  With
 * WQ_ACT_F16, x is fp16 [M][K] (16-byte aligned) and y fp16 [M][N]: every path
 * multiplies fp16 x by exact fp16 code values (q, or q - z; the products are exact in
 * fp32), accumulates in fp32, applies the scales to fp32 sums as for bf16 and rounds y
 * to fp16 (nearest even; beyond 65504 to infinity).
 *   - GEMV (M < 8): the dot2 launch options (rows 4, 8 or 16 without a flag; a flag:
 *     WQ_ERR_UNSUPPORTED).  split_k 0 = the tuned launch of the bf16 layer with its
 *     matrix-core option replaced by the default dot2 launch and its prefetch flag
 *     dropped (waves and rows must then be 0); else as wq_gemv_ex.
 *   - GEMM (M >= 8): per-channel W8 runs tile 2 and the LDS-DMA tiles 9..19 and 24..28
 *     (exact fp16 codes, x as the fp16 operand of the DMA), tiles 3, 4 as 9, 1 as 2, and
 *     5..8, 20..23 as 14; the grouped formats run tile 2 and the LDS-DMA tiles 9..19 and
 *     24..28 (x read as their fp16 operand: no conversion, no row scale, no fallback),
 *     tiles 1, 3, 4 as 9 and 5..8, 20..23 as 14.  The workspace is wq_workspace_size's.
 * wq_moe_linear, wq_lm_head_topk, wq_linear_perm and wq_linear_static take bf16 only.
 * Unknown act: WQ_ERR_INVALID_ARG. */
wq_status wq_linear_act(const wq_weight* w, int act, const void* x, int64_t M, void* y, void* ws,
                        size_t ws_bytes, void* stream);
wq_status wq_gemv_act(const wq_weight* w, int act, const void* x, int64_t M, void* y, int split_k, int waves,
                      int rows, void* ws, size_t ws_bytes, void* stream);
wq_status wq_gemm_act(const wq_weight* w, int act, const void* x, int64_t M, void* y, int tile, void* ws,
                      size_t ws_bytes, void* stream);

/* ------------------------------------------------- the residual epilogue */

/* The layer with a residual added in its epilogue: y = round(x . dequant(W)^T + r), the
 * residual r [M][N] (device, y's type: bf16, or fp16 with WQ_ACT_F16; 2-byte aligned)
 * widened exactly and added to the fp32 result before the one rounding of y (the fused
 * residual of the tileInfer README's "Key Optimizations": the layer's output joins the
 * residual stream without a separate pass over y).  r may be y itself (y += x W^T, in
 * place: every element is read by the thread that writes it, before it writes it); any
 * other overlap of r and y is WQ_ERR_INVALID_ARG, as is a NULL r.  Every path, launch
 * option and tile of wq_linear_act / wq_gemv_act / wq_gemm_act takes it (the residual is
 * added where y is written: by the compute kernel, or by the split-K and tail
 * reductions).  wq_gemv_residual and wq_gemm_residual take the launch explicitly as
 * wq_gemv_act and wq_gemm_act do. */
wq_status wq_linear_residual(const wq_weight* w, int act, const void* x, int64_t M, const void* r, void* y,
                             void* ws, size_t ws_bytes, void* stream);
wq_status wq_gemv_residual(const wq_weight* w, int act, const void* x, int64_t M, const void* r, void* y,
                           int split_k, int waves, int rows, void* ws, size_t ws_bytes, void* stream);
wq_status wq_gemm_residual(const wq_weight* w, int act, const void* x, int64_t M, const void* r, void* y, int tile,
                           void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------- grouped (MoE) layer */

/* The grouped weight-only linear of a mixture-of-experts layer (the shared MoE kernel the
 * Marlin register and launch scheduling benchmark page validates beside its dense one,
 * "Validation and limits"; one WnA16 kernel for every format, SGLang quantization-stack
 * review, Figure 4 comments), optionally with the SiLU gate fused into its epilogue
 * (tileInfer README, "Key Optimizations", fused SiLU gate).
 *
 * E experts of one format and shape (K, N), each packed in the GFX950 layout, are stored
 * one after another: w->qweight, w->scales and w->zeros point to E consecutive packed
 * experts of wq_packed_sizes(fmt, WQ_LAYOUT_GFX950, K, N) bytes each (w describes one
 * expert).  The T rows of x (bf16 [T][K], device, 16-byte aligned) are grouped by expert:
 * expert e owns rows offsets[e] .. offsets[e + 1] - 1, offsets int32 [E + 1] on the
 * device (a routing computed on the device needs no copy to the host; values are
 * clamped into [0, T] and a range that would run backwards is empty, so malformed
 * offsets cannot make the kernel read or write outside x and y).
 *   epilogue WQ_EPILOGUE_NONE:     y bf16 [T][N], y[t] = bf16(x[t] . dequant(W_e)^T);
 *   epilogue WQ_EPILOGUE_SILU_MUL: N = 2 I (the expert's gate rows, then its up rows),
 *     y bf16 [T][I], y[t][j] = bf16(silu(g) * u) with g, u the fp32 sums of gate row j
 *     and up row j, silu(v) = v / (1 + exp(-v)) (g and u never leave the kernel).
 * With E = 1 and offsets {0, T} this is the dense layer (gated or not).  Rows outside
 * every expert's range are not written.
 *
 * Arithmetic as wq_gemv's matrix-core path: exact code values against fp16 x (exact bf16
 * codes against bf16 x where fp16 cannot hold an x exactly), fp32 accumulation, group
 * scales on each group's partial sum, per-channel scales on the finished sum.  An expert
 * is read once per block of 16 of its rows, so the call suits decode-sized batches per
 * expert.  Needs a per-channel or group-128 format (groups of 32 and 64: as the
 * matrix-core GEMV, WQ_ERR_UNSUPPORTED), K % 128 == 0, N % 16 == 0 (N % 32 == 0 gated),
 * T * K and T * N below 2^31 (else WQ_ERR_UNSUPPORTED), 1 <= E <= 65535.  Allocates nothing, needs no
 * workspace, graph-capturable. */
#define WQ_EPILOGUE_NONE 0
#define WQ_EPILOGUE_SILU_MUL 1
wq_status wq_moe_linear(const wq_weight* w, int E, const void* x, const int32_t* offsets, int64_t T, void* y,
                        int epilogue, void* stream);

/* ------------------------------------------- the layer without allocation */

/* wq_linear for callers that cannot allocate device memory or pass a workspace:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  The split-K partials (and, where it fits, the fp16 copy of x of the
 * group-128 GEMM tiles) go to a static scratch array of WQ_STATIC_SCRATCH_BYTES that
 * the library holds on every device it runs on until the process ends; the call itself
 * allocates and frees nothing.  The configuration is the one wq_linear runs (tuned, or
 * the default), so the result is bit-identical to wq_linear given a workspace of
 * wq_workspace_size bytes.  A shape whose configuration needs more partial-sum space
 * than the scratch holds returns WQ_ERR_WORKSPACE (nothing is written); use wq_linear
 * with a workspace there.  The scratch keeps whatever the last call left (no call
 * needs it cleared).  Every call on one device shares that device's scratch, so calls
 * that may overlap on one device (different streams, or threads without ordering) race
 * and must not be issued; calls ordered on one stream are safe.  x, y and the weight as
 * for wq_linear.  The first call on a device looks the scratch address up (no device
 * work, no allocation). */
#define WQ_STATIC_SCRATCH_BYTES (64u << 20)
wq_status wq_linear_static(const wq_weight* w, const void* x, int64_t M, void* y, void* stream);

/* ------------------------------------------------------- LM head + top-k */

/* The LM head followed by top-k sampling in one call ("Fused LM Head + Top-k" and
 * "Distributed Top-k Sampling" in the tileInfer README's feature list: the logits
 * and the sampling in one step, and only the k best logits leave it).  The layer
 * (wq_linear: the GEMV for M < 8) writes bf16 logits [M][N] into the workspace,
 * where they stay; two more kernels select the k best of every row and draw one
 * token from them.
 *
 * Order: larger logit first, equal values by smaller index, -0 == +0, NaN after
 * every number.  Draw: with the kept logits v_1 >= ... >= v_k, weights
 * exp((v_i - v_1) / temperature) in fp32, the token is the first kept one whose
 * running weight exceeds u[m] times the total (the last kept one if none does);
 * temperature 0, or a best logit that is not finite, takes the best; a NaN logit
 * behind a finite best weighs 0.
 *
 * x: bf16 [M][K] (device); u: fp32 [M] (device), the caller's uniform draws in
 * [0, 1); outputs (device): top_vals bf16 [M][k] (the logits' bits), top_idx int32
 * [M][k], best first, and tokens int32 [M].  1 <= k <= min(64, N) and ceil(N / 2048)
 * * k <= 8192 (else WQ_ERR_INVALID_ARG / WQ_ERR_UNSUPPORTED); temperature finite and
 * >= 0; ws (256-byte aligned) of wq_lm_head_topk_workspace_size bytes, else
 * WQ_ERR_WORKSPACE.  Results are bit-identical from run to run. */
wq_status wq_lm_head_topk_workspace_size(const wq_weight* w, int64_t M, int k, size_t* bytes);
wq_status wq_lm_head_topk(const wq_weight* w, const void* x, int64_t M, int k, float temperature,
                          const float* u, void* top_vals, int32_t* top_idx, int32_t* tokens,
                          void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------- full-K activation permutation */

/* The layer on activations gathered along K ("full-K activation permutation" in the
 * Marlin register and launch scheduling benchmark page, "Validation and limits"; the
 * same page counts activation-order index storage in its dense kernel): the weight
 * is stored with its K columns in a permuted order, W'[n][j] = W[n][perm[j]] (pack
 * W' with wq_pack, so its groups are contiguous along the stored order), and
 *   y[m][n] = bf16( sum_j x[m][perm[j]] * dequant(W')[n][j] )  (= x . W^T).
 * One kernel gathers x'[m][j] = x[m][perm[j]] into the workspace, then the layer runs
 * as wq_linear on x' (same dispatch, tuned configurations and rounding: the result is
 * bit-identical to wq_linear on x' given a workspace of wq_workspace_size bytes).
 *
 * x: bf16 [M][K] (device, 2-byte aligned); perm: int32 [K] (device, 4-byte aligned;
 * read as given: an index outside [0, K) reads x as +0, a repeated index is a plain
 * gather); y: bf16 [M][N] (device).  ws (256-byte aligned) of
 * wq_linear_perm_workspace_size bytes (the layer's own workspace, then x'), else
 * WQ_ERR_WORKSPACE.  The caller owns every buffer; nothing is allocated. */
wq_status wq_linear_perm_workspace_size(const wq_weight* w, int64_t M, size_t* bytes);
wq_status wq_linear_perm(const wq_weight* w, const void* x, const int32_t* perm, int64_t M, void* y,
                         void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------ tuner */

/* Choose among measured candidates: the smallest latency wins and a tie goes to
 * the later candidate, as in the split_k loop of "Heuristic: Mit han lab Llm awq
 * Kernel Selection Thresholds" (tinychat/utils/tune.py excerpt, "best >= cur").
 * Host only; returns the index into lat[0..n-1], or -1 if n < 1. */
int wq_tune_pick(const double* lat, int n);

/* Time every candidate for (format, K, N, M) on the current device and store the
 * winner in the tuner cache: for M < 8 every (split_k, waves, rows) triple with
 * split_k in the grid {1,2,4,8,16,32} (those the shape and workspace allow), waves in
 * {1,2,3,4,6,8,12,16} plus the default (capped at wq_gemv_max_waves) and every rows
 * setting; for M >= 8 the GEMM tiles.  The four fastest are then timed a second time,
 * as HIP graph replays of two rotations over the copies (at least 8 calls; captured
 * on a stream the tuner creates and destroys; about `iters` calls timed after 2
 * warm-up replays), and that timing decides among them (where a graph cannot be built
 * the first timing stands).  Each candidate runs `warmup` untimed
 * and `iters` timed calls (the page uses 1000 + 1000), rotating over the n_copies
 * weights (distinct buffers with the same format and shape) so that the weights
 * do not stay cached.  x, y and ws are as for wq_linear.  Writes the chosen split_k
 * (GEMV) or tile (GEMM) to *chosen (host) and, if lat_us is not NULL, the mean
 * microseconds per call of each split_k (its best rows and waves, lat_us[0..5]) or
 * tile (lat_us[tile - 1]) into the WQ_TUNE_LAT_SLOTS entries of lat_us (host; -1
 * for candidates that could not run and for unused slots).  Synchronizes the stream. */
#define WQ_TUNE_LAT_SLOTS 28
wq_status wq_tune(const wq_weight* copies, int n_copies, int64_t M, const void* x, void* y,
                  void* ws, size_t ws_bytes, int warmup, int iters, void* stream, int* chosen,
                  double* lat_us);

/* Tuner cache: entries keyed by (device tag, format, K, N, M, kind), where the
 * device tag is "<gcnArchName>:<compute units>" of the device the entry was tuned
 * on ("" in set/get = the current device).  A GEMV value is split_k | (waves << 8) |
 * (rows << 16), rows possibly | WQ_GEMV_PREFETCH or WQ_GEMV_MFMA (waves or rows 0 = the default for
 * the shape); a GEMM value is a
 * tile id.  get returns WQ_OK and the value, or
 * WQ_ERR_INVALID_ARG when absent.  save/load use a plain text file, one entry per
 * line; load merges into the cache and fails with WQ_ERR_CACHE_IO (leaving the
 * cache unchanged) on a missing or malformed file. */
wq_status wq_tune_cache_set(const char* device_tag, int fmt, int64_t K, int64_t N, int64_t M,
                            int kind, int value);
wq_status wq_tune_cache_get(const char* device_tag, int fmt, int64_t K, int64_t N, int64_t M,
                            int kind, int* value);
wq_status wq_tune_cache_clear(void);
wq_status wq_tune_cache_save(const char* path);
wq_status wq_tune_cache_load(const char* path);

#ifdef __cplusplus
}
#endif

#endif /* WQ_H */
