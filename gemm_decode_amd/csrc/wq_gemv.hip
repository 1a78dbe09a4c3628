// Decode GEMV for 1 <= M <= 7 tokens: y[m][n] = sum_k x[m][k] * dequant(W)[n][k].
//
// Work decomposition (gfx950, wave64), "x-stationary":
//   * K is cut into slices of 64 lanes x one 16-byte code chunk (1024 k for int8,
//     2048 k for uint4).  A wave takes one slice at a time: every lane keeps its
//     chunk of x (all M tokens) in registers and streams the same chunk of each
//     of the workgroup's rows; the row loads of a slice are issued together and,
//     in the gfx950 tiled layout, form one contiguous block (RR x 1 KB per wave).
//   * A workgroup owns RR rows (4, 8 or 16: a whole 16-row tile or a part of one)
//     and one split-K range of slices; its W waves share the slices of that range
//     round-robin.  Few rows per wave means thin waves (few registers, many waves
//     resident to hide memory latency); many rows share each x chunk more widely.
//   * Per lane the RR x M partial sums are reduced across the wave by a butterfly
//     reduce-scatter (after log2(RR) exchange levels lane l holds row l % RR), the
//     W waves' rows meet in LDS and are added in wave order.
//   * split_k > 1 splits the slices across workgroups: each range writes fp32
//     partials to the workspace and a second kernel adds them in range order
//     (deterministic, and no cross-workgroup fence is needed).
//
// In-register dequantisation, exact products with fp32 accumulation:
//   * int8 (gfx950 layout stores u = q + 128): v_perm_b32 places two code bytes
//     under the fp16 exponent byte 0x64, giving the fp16 pair (1024 + u_a, 1024 +
//     u_b) exactly in one instruction, and one packed fp16 add of -1152 leaves the
//     exact codes (q_a, q_b); x is converted to fp16; v_dot2_f32_f16 multiplies.
//   * uint4 (nibbles interleaved by the gfx950 repack, pair i = (q_2i, q_2i+1) at
//     bits 4i and 16 + 4i): word & 0x000F000F | 0x64006400 is the fp16 pair (1024 +
//     q_0, 1024 + q_1), word & 0x00F000F0 | 0x54005400 the fp16 pair (64 + q_2, 64 +
//     q_3) (the nibbles sit on the fp16 units place), and the same on word >> 8 for
//     pairs 2 and 3; one packed fp16 add of -(1024 + z) resp. -(64 + z) leaves the
//     exact q - z; v_dot2_f32_f16 against fp16 x.
//   * Both are exact: every product x q (or x (q - z)) is exact in fp32, so each
//     output carries only the rounding of an fp32 sum and the final bf16 rounding --
//     provided x converts to fp16 exactly, which holds for 0 and 2^-17 <= |x| <=
//     65280.  A slice with any other x takes the bf16 path (codes -> exact bf16 q or
//     q - z, v_dot2_f32_bf16 against bf16 x).
//   * Scales multiply fp32 partial sums (per row at the end for per-channel W8,
//     per chunk for group-128), so codes are never rounded.
//
// Prior art: the tileInfer README ("Key Optimizations": register-only dequantize
// GEMV with 128-bit loads and warp-shuffle reduction, split-K by its kernel's
// name in the project tree), the Marlin benchmark page (intro: FP32 reduction
// scratch for cross-block partial sums) and the awq heuristic page (split_k
// partitions K across thread blocks).  Nothing here follows their code.
#include "wq_internal.h"

namespace wq {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

constexpr int R = kGemvTileRows;  // rows per workgroup tile (16)

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}
__device__ __forceinline__ float dot2_f16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b), c, false);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v;
  v.x = (__bf16)lo;
  v.y = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ float f16_to_f32(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }
__device__ __forceinline__ uint16_t f32_to_bf16(float v) {
  return __builtin_bit_cast(uint16_t, (__bf16)v);  // v_cvt_pk_bf16_f32: nearest even
}
__device__ __forceinline__ uint16_t f32_to_f16(float v) {
  return __builtin_bit_cast(uint16_t, (_Float16)v);  // v_cvt_f16_f32: nearest even
}
// an fp32 result as the output type: bf16, or fp16 for fp16 activations (XF)
template <bool XF>
__device__ __forceinline__ uint16_t f32_to_out(float v) {
  return XF ? f32_to_f16(v) : f32_to_bf16(v);
}
// the fp32 result plus element i of the residual (the output type, widened exactly) when
// there is one: the output is then rounded once.  The residual may be y itself: every
// element is read by the thread that writes it, before it writes it.
template <bool XF>
__device__ __forceinline__ float with_res(float v, const uint16_t* res, size_t i) {
  if (!res) return v;
  return v + (XF ? f16_to_f32(res[i]) : bf16_to_f32(res[i]));
}
// bf16 pair -> fp16 pair (exact in the range described above)
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t b) {
  auto h = __builtin_amdgcn_cvt_pkrtz(__uint_as_float(b << 16), __uint_as_float(b & 0xFFFF0000u));
  return __builtin_bit_cast(uint32_t, h);
}

// fp16 pair + fp16 pair (v_pk_add_f16); exact whenever both sums are representable,
// as for (offset + code) + (-offset).
__device__ __forceinline__ uint32_t add_f16x2(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, a) + __builtin_bit_cast(f16x2_t, b));
}
constexpr uint32_t kF16Minus1152 = 0xE480E480u;  // fp16 pair (-1152, -1152)
// fp16 pair (-v, -v) of a small integer v (exact: v < 2048)
__device__ __forceinline__ uint32_t f16x2_splat_neg(uint32_t v) {
  const uint32_t h = __builtin_bit_cast(uint16_t, (_Float16)(-(float)v));
  return h | (h << 16);
}

// Whether every bf16 value added converts to fp16 exactly: 0, or 2^-17 <= |x| <= 65280
// (a bf16 value has 8 significant bits; fp16 holds them from its subnormal grid 2^-24
// up to its largest finite value, and the next bf16 value after 65280 is 65536).  With
// the sign cleared a bf16 bit pattern orders like its magnitude (Inf and NaN above
// every number): a packed 16-bit running maximum, and a running minimum of the pattern
// minus one (0 wraps to 0xFFFF, so zeros never count as small).
struct F16Exact {
  u16x2_t mx = {0, 0}, mn = {0xFFFF, 0xFFFF};
  __device__ __forceinline__ void add(uint32_t w) {
    const u16x2_t a = __builtin_bit_cast(u16x2_t, w & 0x7FFF7FFFu);
    mx = __builtin_elementwise_max(mx, a);
    mn = __builtin_elementwise_min(mn, a - u16x2_t{1, 1});
  }
  __device__ __forceinline__ bool ok() const {
    return mx.x <= 0x477F && mx.y <= 0x477F && mn.x >= 0x36FF && mn.y >= 0x36FF;
  }
};

// Cross-lane exchange partners.  xor 1 and 2 by DPP quad permutes, xor 4, 8 and 16
// by ds_swizzle (bit-mask mode), xor 32 by ds_bpermute.
template <int J>
__device__ __forceinline__ float xchg(float v) {
  const int i = __builtin_bit_cast(int, v);
  int r;
  if constexpr (J == 1) r = __builtin_amdgcn_mov_dpp(i, 0xB1, 0xF, 0xF, false);
  else if constexpr (J == 2) r = __builtin_amdgcn_mov_dpp(i, 0x4E, 0xF, 0xF, false);
  else if constexpr (J == 4) r = __builtin_amdgcn_ds_swizzle(i, 0x101F);
  else if constexpr (J == 8) r = __builtin_amdgcn_ds_swizzle(i, 0x201F);
  else if constexpr (J == 16) r = __builtin_amdgcn_ds_swizzle(i, 0x401F);
  else r = __shfl_xor(i, 32);
  return __builtin_bit_cast(float, r);
}

// One reduce-scatter level over lanes differing in bit log2(J): values at
// positions 2i and 2i+1 hold rows that differ in the corresponding row bit; the
// lane keeps the one its lane bit selects and adds the partner's copy.
template <int J, int NV, int M, int RR>
__device__ __forceinline__ void rs_level(float (&v)[RR][M], bool hi) {
#pragma unroll
  for (int i = 0; i < NV / 2; ++i)
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const float keep = hi ? v[2 * i + 1][m] : v[2 * i][m];
      const float send = hi ? v[2 * i][m] : v[2 * i + 1][m];
      v[i][m] = keep + xchg<J>(send);
    }
}

template <int FMT>
struct Fmt;
template <>
struct Fmt<WQ_FMT_W8_PC> {
  static constexpr int kChunk = 16;   // k per lane and slice (16 code bytes)
  static constexpr int kXWords = 8;   // bf16 pairs of x per lane and token
};
template <>
struct Fmt<WQ_FMT_W8_G128> {
  static constexpr int kChunk = 16;
  static constexpr int kXWords = 8;
};
template <>
struct Fmt<WQ_FMT_W4_G128> {
  static constexpr int kChunk = 32;
  static constexpr int kXWords = 16;
};

// x words (bf16 pairs) per lane and token of a slice
constexpr int x_words(int fmt) { return fmt == WQ_FMT_W4_G128 ? 16 : 8; }
// Slice prefetch (a launch option): a wave loads its next slice while it multiplies
// the current one, at the price of a second register set of codes and x -- offered
// while that set is small.
constexpr bool prefetch_allowed(int fmt, int RR, int M) { return 4 * RR + M * x_words(fmt) <= 48; }
// Registers a lane needs (estimate: codes, accumulators, x in two forms, addresses,
// the prefetch set) and the largest workgroup whose per-lane budget (512 / ceil(W/4)
// VGPRs) holds them.
constexpr int lane_regs(int fmt, int RR, int M, bool PF) {
  return 40 + 4 * RR + RR * M + 16 * M + (fmt != WQ_FMT_W8_PC ? 8 : 0) + (PF ? 4 * RR + M * x_words(fmt) : 0);
}
constexpr int max_waves_r(int fmt, int RR, int M, bool PF) {
  return lane_regs(fmt, RR, M, PF) <= 118 ? 16 : lane_regs(fmt, RR, M, PF) <= 236 ? 8 : 4;
}

// grid = (16-row tiles x sub-tiles of RR rows, split_k); block = 64 * W threads.
// XF: x and y in fp16 (fp16 activations): x is already the fp16 operand, so the
// conversion and its exactness check drop out, and y is rounded to fp16.
template <int FMT, int M, int RR, bool PF, bool XF = false>
__global__ __launch_bounds__(64 * max_waves_r(FMT, RR, M, PF)) void gemv_kernel(
    const uint8_t* __restrict__ qw, const uint16_t* __restrict__ scales,
    const uint8_t* __restrict__ zeros, const uint16_t* __restrict__ x, uint16_t* y,
    float* __restrict__ part, int K, int N, int gshift, const uint16_t* res) {
  using F = Fmt<FMT>;
  constexpr int kSlice = 64 * F::kChunk;
  constexpr bool kW4 = FMT == WQ_FMT_W4_G128;
  constexpr int MAXW = max_waves_r(FMT, RR, M, PF);
  constexpr int NSUB = R / RR;
  __shared__ float red[MAXW][M * RR];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int W = blockDim.x >> 6;
  const int tile = blockIdx.x / NSUB, sub = blockIdx.x % NSUB;
  const int n0 = tile * R + sub * RR;
  if (n0 >= N) return;  // the whole workgroup leaves together
  const int s = blockIdx.y, S = gridDim.y;
  const int T = (K + kSlice - 1) / kSlice;
  const int sl0 = (int)(((int64_t)s * T) / S), sl1 = (int)(((int64_t)(s + 1) * T) / S);
  const int G = K >> gshift;  // groups per row: 2^gshift k each (32, 64 or 128; a lane's chunk lies in one)
  const size_t row_bytes = kW4 ? (size_t)K / 2 : (size_t)K;
  // tile base in the gfx950 code layout and its row count (the last tile may be short)
  const uint8_t* tile_base = qw + (size_t)tile * R * row_bytes;
  const int nr = min(R, N - tile * R);

  float acc[RR][M];
#pragma unroll
  for (int r = 0; r < RR; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] = 0.f;

  // Full slices of a full tile (every row a whole 1 KB, no row past N) take the fast
  // form: wave-uniform slice base + a 32-bit lane offset + r KB, so the loads need no
  // 64-bit address arithmetic; the ragged last slice and a short last tile take the
  // general form.
  const int wu = __builtin_amdgcn_readfirstlane(wave);
  const int t_full = nr == R ? (int)(row_bytes / kSliceBytes) : 0;  // slices with whole 1 KB rows
  const uint32_t rlane = (uint32_t)(sub * RR) * kSliceBytes + lane * 16;
  const uint32_t xlane = (uint32_t)lane * F::kChunk * 2;  // byte offset of this lane's x chunk in a slice
  // The uint4 nibble masks and the fp16 1024.0 / 64.0 pairs live in registers the
  // compiler cannot see through, so each code pair is one v_and_or_b32 rather than a
  // separate and/or with two literal operands.
  uint32_t nib_mask = 0x000F000Fu, f16_1024 = 0x64006400u, nib_mask_hi = 0x00F000F0u, f16_64 = 0x54005400u;
  if constexpr (kW4) asm volatile("" : "+v"(nib_mask), "+v"(f16_1024), "+v"(nib_mask_hi), "+v"(f16_64));

  // The arithmetic of one slice, given its codes (RR rows) and x chunk.
  auto slice_math = [&](const uint4* cw, const uint32_t (*xb)[F::kXWords], int kk) {
    const int g = kk >> gshift;
    uint32_t sw[RR / 2];  // RR 16-bit scales of this sub-tile's rows for group g
    uint32_t zw = 0;      // RR 4-bit zero-points
    if constexpr (FMT != WQ_FMT_W8_PC) {
      const uint16_t* sp = scales + ((size_t)tile * G + g) * R + sub * RR;
      if constexpr (RR == 16) {
        const uint4 a = reinterpret_cast<const uint4*>(sp)[0], b = reinterpret_cast<const uint4*>(sp)[1];
        sw[0] = a.x; sw[1] = a.y; sw[2] = a.z; sw[3] = a.w; sw[4] = b.x; sw[5] = b.y; sw[6] = b.z; sw[7] = b.w;
      } else if constexpr (RR == 8) {
        const uint4 a = reinterpret_cast<const uint4*>(sp)[0];
        sw[0] = a.x; sw[1] = a.y; sw[2] = a.z; sw[3] = a.w;
      } else {
        const uint2 a = reinterpret_cast<const uint2*>(sp)[0];
        sw[0] = a.x; sw[1] = a.y;
      }
    }
    uint32_t zw_hi = 0;
    if constexpr (kW4) {
      const uint8_t* zp = zeros + ((size_t)tile * G + g) * (R / 2) + sub * (RR / 2);
      if constexpr (RR == 16) {
        const uint2 a = *reinterpret_cast<const uint2*>(zp);
        zw = a.x;
        zw_hi = a.y;
      } else if constexpr (RR == 8) {
        zw = *reinterpret_cast<const uint32_t*>(zp);
      } else {
        zw = *reinterpret_cast<const uint16_t*>(zp);
      }
    }
    auto scale_of = [&](int r) -> uint16_t {
      const uint32_t word = sw[r >> 1];
      return (uint16_t)((r & 1) ? (word >> 16) : (word & 0xFFFFu));
    };
    auto zero_of = [&](int r) -> uint32_t { return ((r < 8 ? zw : zw_hi) >> (4 * (r & 7))) & 0xFu; };

    // Does every x of the slice convert to fp16 exactly (see F16Exact)?  Otherwise the
    // whole wave takes the bf16 path for this slice.  (fp16 x: it is the operand.)
    bool exact_path = false;
    if constexpr (!XF) {
      F16Exact fx;
#pragma unroll
      for (int m = 0; m < M; ++m)
#pragma unroll
        for (int i = 0; i < F::kXWords; ++i) fx.add(xb[m][i]);
      exact_path = __builtin_amdgcn_ballot_w64(!fx.ok()) != 0;
    }

    if constexpr (!kW4) {
      // ---- int8: fp16 (1024 + u) by v_perm_b32, minus 1152 by one packed fp16 add: the
      // exact code q, against fp16 x
      if (!exact_path) {
        uint32_t xh[M][8];
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
          for (int i = 0; i < 8; ++i) xh[m][i] = XF ? xb[m][i] : bf16x2_to_f16x2(xb[m][i]);
#pragma unroll
        for (int r = 0; r < RR; ++r) {
          const uint32_t d[4] = {cw[r].x, cw[r].y, cw[r].z, cw[r].w};
          uint32_t hp[8];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            hp[2 * j] = add_f16x2(__builtin_amdgcn_perm(0x64646464u, d[j], 0x04010400u), kF16Minus1152);
            hp[2 * j + 1] = add_f16x2(__builtin_amdgcn_perm(0x64646464u, d[j], 0x04030402u), kF16Minus1152);
          }
          if constexpr (FMT == WQ_FMT_W8_PC) {
#pragma unroll
            for (int m = 0; m < M; ++m)
#pragma unroll
              for (int i = 0; i < 8; ++i) acc[r][m] = dot2_f16(hp[i], xh[m][i], acc[r][m]);
          } else {
            const float sc = bf16_to_f32(scale_of(r));
#pragma unroll
            for (int m = 0; m < M; ++m) {
              float t = 0.f;
#pragma unroll
              for (int i = 0; i < 8; ++i) t = dot2_f16(hp[i], xh[m][i], t);
              acc[r][m] = fmaf(sc, t, acc[r][m]);
            }
          }
        }
      } else {
        // bf16 path: signed code -> fp32 -> bf16 pairs, against bf16 x
#pragma unroll
        for (int r = 0; r < RR; ++r) {
          const uint32_t d[4] = {cw[r].x ^ 0x80808080u, cw[r].y ^ 0x80808080u, cw[r].z ^ 0x80808080u,
                                 cw[r].w ^ 0x80808080u};
          uint32_t bp[8];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            bp[2 * j] = pack_bf16x2((float)(int8_t)(d[j] & 0xFFu), (float)(int8_t)((d[j] >> 8) & 0xFFu));
            bp[2 * j + 1] = pack_bf16x2((float)(int8_t)((d[j] >> 16) & 0xFFu), (float)(int8_t)(d[j] >> 24));
          }
          const float sc = (FMT == WQ_FMT_W8_G128) ? bf16_to_f32(scale_of(r)) : 1.f;
#pragma unroll
          for (int m = 0; m < M; ++m) {
            float t = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) t = dot2_bf16(bp[i], xb[m][i], t);
            acc[r][m] = fmaf(sc, t, acc[r][m]);
          }
        }
      }
    } else if (!exact_path) {
      // ---- uint4 group-128.  Of each word's four nibble pairs, those at bits (0, 16) and,
      // after one shift by 8, (8, 24) go under the fp16 1024.0 pattern (1024 + q), those
      // at (4, 20) and (12, 28) under the fp16 64.0 pattern (64 + q: the nibble sits on
      // the units place); one packed fp16 add of -(1024 + z) resp. -(64 + z) leaves the
      // exact q - z, against fp16 x.
      uint32_t xh[M][16];
#pragma unroll
      for (int m = 0; m < M; ++m)
#pragma unroll
        for (int i = 0; i < 16; ++i) xh[m][i] = XF ? xb[m][i] : bf16x2_to_f16x2(xb[m][i]);
#pragma unroll
      for (int r = 0; r < RR; ++r) {
        const float sc = f16_to_f32(scale_of(r));
        const uint32_t z = zero_of(r);
        const uint32_t off_a = f16x2_splat_neg(1024u + z), off_b = f16x2_splat_neg(64u + z);
        const uint32_t words[4] = {cw[r].x, cw[r].y, cw[r].z, cw[r].w};
        float t[M];
#pragma unroll
        for (int m = 0; m < M; ++m) t[m] = 0.f;
#pragma unroll
        for (int wi = 0; wi < 4; ++wi) {
          const uint32_t w = words[wi], w8 = w >> 8;
          const uint32_t p0 = add_f16x2((w & nib_mask) | f16_1024, off_a);
          const uint32_t p1 = add_f16x2((w & nib_mask_hi) | f16_64, off_b);
          const uint32_t p2 = add_f16x2((w8 & nib_mask) | f16_1024, off_a);
          const uint32_t p3 = add_f16x2((w8 & nib_mask_hi) | f16_64, off_b);
#pragma unroll
          for (int m = 0; m < M; ++m) {
            t[m] = dot2_f16(p0, xh[m][4 * wi], t[m]);
            t[m] = dot2_f16(p1, xh[m][4 * wi + 1], t[m]);
            t[m] = dot2_f16(p2, xh[m][4 * wi + 2], t[m]);
            t[m] = dot2_f16(p3, xh[m][4 * wi + 3], t[m]);
          }
        }
#pragma unroll
        for (int m = 0; m < M; ++m) acc[r][m] = fmaf(sc, t[m], acc[r][m]);
      }
    } else {
      // ---- uint4 group-128, exact path: bf16(q - z) pairs
#pragma unroll
      for (int r = 0; r < RR; ++r) {
        const float sc = f16_to_f32(scale_of(r));
        const float z = (float)zero_of(r);
        const uint32_t words[4] = {cw[r].x, cw[r].y, cw[r].z, cw[r].w};
        float t[M];
#pragma unroll
        for (int m = 0; m < M; ++m) t[m] = 0.f;
#pragma unroll
        for (int wi = 0; wi < 4; ++wi)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t p = pack_bf16x2((float)((words[wi] >> (4 * i)) & 0xFu) - z,
                                           (float)((words[wi] >> (16 + 4 * i)) & 0xFu) - z);
#pragma unroll
            for (int m = 0; m < M; ++m) t[m] = dot2_bf16(p, xb[m][4 * wi + i], t[m]);
          }
#pragma unroll
        for (int m = 0; m < M; ++m) acc[r][m] = fmaf(sc, t[m], acc[r][m]);
      }
    }
  };

  // Full slices: no bounds logic, 32-bit lane offsets from wave-uniform bases.  A wave
  // with several slices loads the next one while it multiplies the current one (two
  // register sets with fixed roles: copying a set would wait for its loads).
  auto load_full = [&](uint4* cw, uint32_t (*xb)[F::kXWords], int sl) {
    // (a tile is at most 16 x 2^22 bytes: 32-bit scalar offsets)
    const uint8_t* sblock = tile_base + (uint32_t)(nr * kSliceBytes) * (uint32_t)sl;
#pragma unroll
    for (int r = 0; r < RR; ++r) cw[r] = load_stream16(sblock + rlane + r * kSliceBytes);
    const uint8_t* xs_base = reinterpret_cast<const uint8_t*>(x) + (uint32_t)sl * (uint32_t)(kSlice * 2);
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const uint4* xp = reinterpret_cast<const uint4*>(xs_base + (uint32_t)m * (uint32_t)K * 2 + xlane);
#pragma unroll
      for (int j = 0; j < F::kXWords / 4; ++j) {
        const uint4 v = xp[j];
        xb[m][4 * j + 0] = v.x;
        xb[m][4 * j + 1] = v.y;
        xb[m][4 * j + 2] = v.z;
        xb[m][4 * j + 3] = v.w;
      }
    }
  };
  int sl = sl0 + wu;
  const int sl_end = min(sl1, t_full);
  if constexpr (!PF) {
    for (; sl < sl_end; sl += W) {
      uint4 cw[RR];
      uint32_t xb[M][F::kXWords];
      load_full(cw, xb, sl);
      slice_math(cw, xb, sl * kSlice + lane * F::kChunk);
    }
  } else if (sl < sl_end) {
    // Every load of the next slice is unconditional inside its block (a load under a
    // branch would make the compiler wait for it before touching the current slice).
    uint4 ca[RR], cb[RR];
    uint32_t xa[M][F::kXWords], xbb[M][F::kXWords];
    load_full(ca, xa, sl);
    for (;;) {
      if (sl + W >= sl_end) {
        slice_math(ca, xa, sl * kSlice + lane * F::kChunk);
        sl += W;
        break;
      }
      load_full(cb, xbb, sl + W);
      slice_math(ca, xa, sl * kSlice + lane * F::kChunk);
      sl += W;
      if (sl + W >= sl_end) {
        slice_math(cb, xbb, sl * kSlice + lane * F::kChunk);
        sl += W;
        break;
      }
      load_full(ca, xa, sl + W);
      slice_math(cb, xbb, sl * kSlice + lane * F::kChunk);
      sl += W;
    }
  }
  // the ragged last slice, or every slice of a short last tile: general addressing
  for (; sl < sl1; sl += W) {
    const int k = sl * kSlice + lane * F::kChunk;
    const bool valid = k < K;
    const int kk = valid ? k : 0;
    const int wsl = (int)min((size_t)kSliceBytes, row_bytes - (size_t)sl * kSliceBytes);  // bytes per row
    const uint8_t* sbase = tile_base + (size_t)nr * kSliceBytes * sl + (valid ? lane * 16 : 0);
    uint4 cw[RR];
#pragma unroll
    for (int r = 0; r < RR; ++r)
      cw[r] = load_stream16(sbase + (size_t)min(sub * RR + r, nr - 1) * wsl);
    uint32_t xb[M][F::kXWords];
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const uint4* xp = reinterpret_cast<const uint4*>(x + (size_t)m * K + kk);
#pragma unroll
      for (int j = 0; j < F::kXWords / 4; ++j) {
        const uint4 a = xp[j];
        xb[m][4 * j + 0] = valid ? a.x : 0u;
        xb[m][4 * j + 1] = valid ? a.y : 0u;
        xb[m][4 * j + 2] = valid ? a.z : 0u;
        xb[m][4 * j + 3] = valid ? a.w : 0u;
      }
    }
    slice_math(cw, xb, kk);
  }
  // ---- wave reduce-scatter: afterwards lane l holds row (l % RR), all M tokens
  rs_level<1, RR, M>(acc, lane & 1);
  if constexpr (RR >= 4) rs_level<2, RR / 2, M>(acc, lane & 2);
  if constexpr (RR >= 8) rs_level<4, RR / 4, M>(acc, lane & 4);
  if constexpr (RR >= 16) rs_level<8, RR / 8, M>(acc, lane & 8);
#pragma unroll
  for (int m = 0; m < M; ++m) {
    if constexpr (RR <= 4) acc[0][m] += xchg<4>(acc[0][m]);
    if constexpr (RR <= 8) acc[0][m] += xchg<8>(acc[0][m]);
    acc[0][m] += xchg<16>(acc[0][m]);
    acc[0][m] += xchg<32>(acc[0][m]);
  }

  const int row = lane % RR, n = n0 + row;
  float v[M];
  if (W == 1) {
#pragma unroll
    for (int m = 0; m < M; ++m) v[m] = acc[0][m];
  } else {
    if (lane < RR) {
#pragma unroll
      for (int m = 0; m < M; ++m) red[wave][m * RR + row] = acc[0][m];
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float a = 0.f;
      for (int w = 0; w < W; ++w) a += red[w][m * RR + row];
      v[m] = a;
    }
  }
  if (lane < RR && n < N) {
    if (S == 1) {
      const float sc = (FMT == WQ_FMT_W8_PC) ? bf16_to_f32(scales[n]) : 1.f;
#pragma unroll
      for (int m = 0; m < M; ++m)
        y[(size_t)m * N + n] = f32_to_out<XF>(with_res<XF>(sc * v[m], res, (size_t)m * N + n));
    } else {
#pragma unroll
      for (int m = 0; m < M; ++m) part[((size_t)s * M + m) * N + n] = v[m];
    }
  }
}

// y[m][n] = bf16(scale[n] * sum_s part[s][m][n]) (fp16 with XF), ranges added in order.
template <int FMT, bool XF = false>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part,
                                                              const uint16_t* __restrict__ scales,
                                                              uint16_t* y, int M,
                                                              int N, int S, const uint16_t* res) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t MN = (int64_t)M * N;
  if (i >= MN) return;
  float v = 0.f;
  for (int s = 0; s < S; ++s) v += part[(int64_t)s * MN + i];
  const int n = (int)(i % N);
  const float sc = (FMT == WQ_FMT_W8_PC) ? bf16_to_f32(scales[n]) : 1.f;
  y[i] = f32_to_out<XF>(with_res<XF>(sc * v, res, (size_t)i));
}

// ---------------------------------------------------------------------------------
// Matrix-core GEMV (launch option: rows = 16 NB | kGemvMfma).
//
// The multiply-adds of the decode GEMV go to v_mfma_f32_16x16x32 (bf16 and fp16)
// instead of v_dot2, which leaves the VALU the code extraction and, for group-128,
// one fold per group; the cost no longer grows with the token count M.  Operand
// layouts of the 16x16x32 matrix instructions: lane l holds A[row l % 16][k 8 (l / 16)
// .. +7] and B[k 8 (l / 16) .. +7][column l % 16] and receives D[rows 4 (l / 16) .. +3]
// [column l % 16].  Here A is x (row = token; rows >= M repeat token M - 1 and their
// D rows are never read) and B is 16 weight rows of one gfx950 tile.  K is walked in
// units of 128 k (a group of the group-128 formats): lane l takes k = 32 (l / 16) ..
// +31 of the unit in tile row l % 16 -- 16 code bytes (uint4: at 64 u' + 16 (l / 16)
// of its 1 KB row slice, u' the unit within the slice) or 32 (int8: at 128 u' + 32 (l
// / 16)) -- and x at the same k; instruction s (0..3) of a unit contracts k = 32 (l /
// 16) + 8 s + 0..7 in A and B alike.
//
// Codes become exact fp16 values as in the dot2 path: int8 (stored u = q + 128) by
// v_perm_b32 under the fp16 exponent byte 0x64 (1024 + u) and one packed fp16 add of
// -1152; uint4 pairs at bits (0, 16) and, after a shift by 8, (8, 24) under the fp16
// 1024.0 pattern, pairs at (4, 20) and (12, 28) under the fp16 64.0 pattern, then one
// packed fp16 add of -(1024 + z) resp. -(64 + z): the exact q - z.  x is converted to
// fp16, so every product is exact and accumulates in fp32; a unit with an x that
// does not convert to fp16 exactly (see F16Exact) takes exact bf16 codes (q or q - z)
// against bf16 x.  Group-128 scales each group's partial and adds it up.  A ragged
// last unit (int8 with K % 128 != 0) masks the lanes past K.
constexpr int kMmaMaxWaves = 8;

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mma_bf16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mma_f16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}
// exact bf16 pairs of four signed codes stored as u = q + 128
__device__ __forceinline__ void i8_word_to_bf16(uint32_t d, uint32_t& lo, uint32_t& hi) {
  d ^= 0x80808080u;
  lo = pack_bf16x2((float)(int8_t)(d & 0xFFu), (float)(int8_t)((d >> 8) & 0xFFu));
  hi = pack_bf16x2((float)(int8_t)((d >> 16) & 0xFFu), (float)(int8_t)(d >> 24));
}

// LX (x in LDS): the workgroup first converts its K range of x to fp16 in LDS (M x 128 k
// per unit, uint4 operands in their lo / hi order) with one flag per unit that is set
// when some x of the unit does not convert exactly; the waves then read their A
// operands from LDS instead of converting and checking x for every unit, and load the
// next unit's codes while multiplying the current one.  Chosen by the launcher when the
// fp16 x fits kLxMaxBytes.
constexpr int kLxMaxBytes = 64 * 1024;
inline int lx_bytes(int M, int units) { return M * units * 256 + ((units + 15) & ~15); }

// M: the tokens (1..7), or kMmaTokens for a token count Mt of 8..kMmaTokens chosen at run
// time (the GEMM's few-token tiles): the A operand holds 16 tokens, so a lane's x row is
// its own token and the cost barely depends on M.
template <int FMT, int M, int NB, bool LX>
__global__ __launch_bounds__(64 * kMmaMaxWaves) void gemv_mma_kernel(
    const uint8_t* __restrict__ qw, const uint16_t* __restrict__ scales, const uint8_t* __restrict__ zeros,
    const uint16_t* __restrict__ x, uint16_t* y, float* __restrict__ part, int K, int N, int Mt,
    const uint16_t* res) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lx_mem[];
  constexpr bool kW4 = FMT == WQ_FMT_W4_G128, kGrouped = FMT != WQ_FMT_W8_PC;
  constexpr int MI = M < 4 ? M : 4;             // accumulator rows a lane keeps (token 4 (l / 16) + i, i < MI)
  const int Mr = M <= kGemvMaxM ? M : Mt;       // tokens
  constexpr int kUnitBytes = kW4 ? 64 : 128;    // code bytes per row and 128-k unit
  constexpr int kUnitsPerSlice = kSliceBytes / kUnitBytes;
  constexpr int CL = kW4 ? 1 : 2;               // 16-byte code loads per lane, tile and unit
  __shared__ float red[kMmaMaxWaves][NB][M][16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, W = blockDim.x >> 6;
  const int wu = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t ln = lane & 15, lk = lane >> 4;
  const int T16 = (N + 15) >> 4;
  const int tile0 = blockIdx.x * NB;
  const int s = blockIdx.y, S = gridDim.y;
  const int U = (K + kGroup - 1) / kGroup, G = K / kGroup;
  const int u0 = (int)((int64_t)s * U / S), u1 = (int)((int64_t)(s + 1) * U / S);
  const uint32_t row_bytes = kW4 ? (uint32_t)K / 2 : (uint32_t)K;

  // Per tile: wave-uniform bases (codes, group scales, zero-points) and this lane's
  // row.  Loads take a uniform base plus a 32-bit lane offset.
  const uint8_t* tbase[NB];
  const uint8_t* sbase[NB];
  const uint8_t* zbase[NB];
  uint32_t nr1k[NB], rsel[NB];
#pragma unroll
  for (int t = 0; t < NB; ++t) {
    const int tt = min(tile0 + t, T16 - 1);  // tiles past the end repeat the last (not stored)
    const int nr = min(16, N - 16 * tt);
    tbase[t] = qw + (size_t)tt * 16 * row_bytes;
    sbase[t] = reinterpret_cast<const uint8_t*>(scales + (kGrouped ? (size_t)tt * G * 16 : 0));
    zbase[t] = kW4 ? zeros + (size_t)tt * G * 8 : nullptr;
    nr1k[t] = (uint32_t)nr * kSliceBytes;
    rsel[t] = min(ln, (uint32_t)nr - 1u);
  }
  const uint8_t* xb8 = reinterpret_cast<const uint8_t*>(x);
  const uint32_t xrow = min(ln, (uint32_t)Mr - 1u) * (uint32_t)K * 2u;  // byte offset of this lane's token
  // metadata of row ln within the 32-bit words that hold it: its fp16/bf16 scale is half
  // ln & 1 of a word, its zero-point nibble ln & 7 of one
  const uint32_t sshift = 16 * (ln & 1), zshift = 4 * (ln & 7);
  uint32_t m_lo = 0x000F000Fu, m_hi = 0x00F000F0u, mag_a = 0x64006400u, mag_h = 0x54005400u;
  if constexpr (kW4) asm volatile("" : "+v"(m_lo), "+v"(m_hi), "+v"(mag_a), "+v"(mag_h));

  f32x4_t acc[NB];  // group-128: scaled sums; per-channel: raw sums of x q
#pragma unroll
  for (int t = 0; t < NB; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int nu = u1 - u0;                      // LX: units of this workgroup's K range
  uint8_t* lx_flag = lx_mem + Mr * nu * 256;   // LX: per unit, 1 if some x is not fp16-exact


  // One unit's operands (32-bit fields only, so that the set stays in registers).
  struct Set {
    u32x4_t c[NB][CL];
    uint4 xv[4];
    uint32_t sv[NB], zb[NB];
  };
  // this lane's 32 x values of unit u (token min(l % 16, M - 1)); zero past K
  auto load_x = [&](uint4 (&xv)[4], int u) {
    const uint32_t k0 = 128u * (uint32_t)u + 32u * lk;
    if (kW4 || 128 * (u + 1) <= K) {
      const uint4* xp = reinterpret_cast<const uint4*>(xb8 + (xrow + 2u * k0));
#pragma unroll
      for (int j = 0; j < 4; ++j) xv[j] = xp[j];
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t k = k0 + 8u * j;
        const bool ok = k + 8u <= (uint32_t)K;
        const uint4 v = *reinterpret_cast<const uint4*>(xb8 + (xrow + 2u * (ok ? k : 0u)));
        xv[j] = ok ? v : make_uint4(0u, 0u, 0u, 0u);
      }
    }
  };
  auto load = [&](Set& st, int u) {
    const uint32_t sl = (uint32_t)u / kUnitsPerSlice, ui = (uint32_t)u % kUnitsPerSlice;
    const uint32_t wsl = min((uint32_t)kSliceBytes, row_bytes - (uint32_t)kSliceBytes * sl);
    const uint32_t k0 = 128u * (uint32_t)u + 32u * lk;  // this lane's first k
    if (kW4 || 128 * (u + 1) <= K) {                     // a whole unit (wave-uniform)
#pragma unroll
      for (int t = 0; t < NB; ++t)
#pragma unroll
        for (int c = 0; c < CL; ++c)
          st.c[t][c] = __builtin_bit_cast(
              u32x4_t, load_stream16(tbase[t] + nr1k[t] * sl +
                                     (__umul24(rsel[t], wsl) + kUnitBytes * ui + (kW4 ? 16u : 32u) * lk + 16u * c)));
      if constexpr (!LX) load_x(st.xv, u);
    } else {
      // the ragged last unit: chunks past K load any in-bounds chunk, their x is zero
#pragma unroll
      for (int t = 0; t < NB; ++t)
#pragma unroll
        for (int c = 0; c < CL; ++c) {
          const bool ok = k0 + 16u * c + 16u <= (uint32_t)K;
          const uint32_t off = ok ? kUnitBytes * ui + 32u * lk + 16u * c : 0u;
          st.c[t][c] = __builtin_bit_cast(u32x4_t, load_stream16(tbase[t] + nr1k[t] * sl +
                                                                 (__umul24(rsel[t], wsl) + off)));
        }
      if constexpr (!LX) load_x(st.xv, u);
    }
    if constexpr (kGrouped) {
      // whole aligned words: a loaded byte or half would be re-extended where the loop
      // carries it, and that wait would drain the next unit's loads as well
      const uint32_t soff = 32u * (uint32_t)u + 4u * (ln >> 1), zoff = 8u * (uint32_t)u + 4u * (ln >> 3);
#pragma unroll
      for (int t = 0; t < NB; ++t) {
        st.sv[t] = *reinterpret_cast<const uint32_t*>(sbase[t] + soff);
        st.zb[t] = kW4 ? *reinterpret_cast<const uint32_t*>(zbase[t] + zoff) : 0u;
      }
    }
  };
  // LX: the first unit's code loads go out first, so that their latency overlaps the
  // conversion of x into LDS
  const int first = u0 + wu;
  const int n_my = first < u1 ? (u1 - first + W - 1) / W : 0;
  Set sa, sb;
  if constexpr (LX) {
    if (n_my > 0) load(sa, first);
  }
  if constexpr (LX) {
    for (int i = threadIdx.x; i < nu; i += blockDim.x) lx_flag[i] = 0;
    __syncthreads();
    // chunk c: token m, unit uu, 8 values j of the unit (k = 128 (u0 + uu) + 8 j)
    for (int c = threadIdx.x; c < Mr * nu * 16; c += blockDim.x) {
      const int m = c / (nu * 16), r = c - m * nu * 16, uu = r >> 4, j = r & 15;
      const int k = 128 * (u0 + uu) + 8 * j;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (k + 8 <= K) v = *reinterpret_cast<const uint4*>(x + (size_t)m * K + k);
      F16Exact fx;
      fx.add(v.x);
      fx.add(v.y);
      fx.add(v.z);
      fx.add(v.w);
      if (!fx.ok()) lx_flag[uu] = 1;
      const uint32_t h0 = bf16x2_to_f16x2(v.x), h1 = bf16x2_to_f16x2(v.y), h2 = bf16x2_to_f16x2(v.z),
                     h3 = bf16x2_to_f16x2(v.w);
      uint8_t* dst = lx_mem + (size_t)(m * nu + uu) * 256;
      if constexpr (kW4) {
        // word i of a 32-k block (pair k = 2i, 2i + 1) sits at i / 2 (i even: the pairs
        // the 1024.0 pattern meets) or 8 + (i - 1) / 2 (odd: the 64.0 pattern's)
        uint32_t* blk = reinterpret_cast<uint32_t*>(dst + 64 * (j >> 2));
        const int jp = j & 3;
        *reinterpret_cast<uint2*>(blk + 2 * jp) = make_uint2(h0, h2);
        *reinterpret_cast<uint2*>(blk + 8 + 2 * jp) = make_uint2(h1, h3);
      } else {
        *reinterpret_cast<uint4*>(dst + 16 * j) = make_uint4(h0, h1, h2, h3);
      }
    }
    __syncthreads();
  }

  auto compute = [&](const Set& st, int u) {
    uint4 xv[4];
    bool exact;
    const u32x4_t* xa = nullptr;  // LX: this lane's four fp16 A operands in LDS
    if constexpr (LX) {
      exact = __builtin_amdgcn_readfirstlane(lx_flag[u - u0]) != 0;
      xa = reinterpret_cast<const u32x4_t*>(lx_mem + (size_t)(min(ln, (uint32_t)Mr - 1u) * nu + (u - u0)) * 256 +
                                            64 * lk);
      if (exact) load_x(xv, u);
    } else {
      xv[0] = st.xv[0];
      xv[1] = st.xv[1];
      xv[2] = st.xv[2];
      xv[3] = st.xv[3];
      // does every x of the unit convert to fp16 exactly (see the dot2 path)?
      F16Exact fx;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        fx.add(xv[j].x);
        fx.add(xv[j].y);
        fx.add(xv[j].z);
        fx.add(xv[j].w);
      }
      exact = __builtin_amdgcn_ballot_w64(!fx.ok()) != 0;
    }
    // group-128: the unit's contribution d[t] to each tile, times the group scale
    auto fold1 = [&](int t, const f32x4_t& d) {
      const uint16_t sh = (uint16_t)(st.sv[t] >> sshift);
      const float sc = kW4 ? f16_to_f32(sh) : bf16_to_f32(sh);
#pragma unroll
      for (int i = 0; i < MI; ++i) acc[t][i] = fmaf(sc, d[i], acc[t][i]);
    };
    auto fold = [&](const f32x4_t (&d)[NB]) {
#pragma unroll
      for (int t = 0; t < NB; ++t) fold1(t, d[t]);
    };
    if (!exact) {
      if constexpr (kW4) {
        u32x4_t a_lo0, a_lo1, a_hi0, a_hi1;
        if constexpr (LX) {
          a_lo0 = xa[0];
          a_lo1 = xa[1];
          a_hi0 = xa[2];
          a_hi1 = xa[3];
        } else {
          a_lo0 = u32x4_t{bf16x2_to_f16x2(xv[0].x), bf16x2_to_f16x2(xv[0].z), bf16x2_to_f16x2(xv[1].x),
                          bf16x2_to_f16x2(xv[1].z)};
          a_lo1 = u32x4_t{bf16x2_to_f16x2(xv[2].x), bf16x2_to_f16x2(xv[2].z), bf16x2_to_f16x2(xv[3].x),
                          bf16x2_to_f16x2(xv[3].z)};
          a_hi0 = u32x4_t{bf16x2_to_f16x2(xv[0].y), bf16x2_to_f16x2(xv[0].w), bf16x2_to_f16x2(xv[1].y),
                          bf16x2_to_f16x2(xv[1].w)};
          a_hi1 = u32x4_t{bf16x2_to_f16x2(xv[2].y), bf16x2_to_f16x2(xv[2].w), bf16x2_to_f16x2(xv[3].y),
                          bf16x2_to_f16x2(xv[3].w)};
        }
        u32x4_t b[4][NB];  // the four B operands of each tile: exact fp16 q - z
#pragma unroll
        for (int t = 0; t < NB; ++t) {
          const uint32_t z = (st.zb[t] >> zshift) & 15u;
          // fp16 pairs -(1024 + z) = 0xE400 + z and -(64 + z) = 0xD400 + 16 z
          const uint32_t off_a = 0xE400E400u + z * 0x10001u, off_b = 0xD400D400u + z * 0x100010u;
          uint32_t lo[4], lo8[4], hi[4], hi8[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t w = st.c[t][0][q], w8 = w >> 8;
            lo[q] = add_f16x2((w & m_lo) | mag_a, off_a);
            hi[q] = add_f16x2((w & m_hi) | mag_h, off_b);
            lo8[q] = add_f16x2((w8 & m_lo) | mag_a, off_a);
            hi8[q] = add_f16x2((w8 & m_hi) | mag_h, off_b);
          }
          b[0][t] = u32x4_t{lo[0], lo8[0], lo[1], lo8[1]};
          b[1][t] = u32x4_t{lo[2], lo8[2], lo[3], lo8[3]};
          b[2][t] = u32x4_t{hi[0], hi8[0], hi[1], hi8[1]};
          b[3][t] = u32x4_t{hi[2], hi8[2], hi[3], hi8[3]};
        }
        f32x4_t d[NB];
#pragma unroll
        for (int t = 0; t < NB; ++t) d[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        // the four products, tiles interleaved so that no instruction waits for the previous
#pragma unroll
        for (int t = 0; t < NB; ++t) d[t] = mma_f16(a_lo0, b[0][t], d[t]);
#pragma unroll
        for (int t = 0; t < NB; ++t) d[t] = mma_f16(a_lo1, b[1][t], d[t]);
#pragma unroll
        for (int t = 0; t < NB; ++t) d[t] = mma_f16(a_hi0, b[2][t], d[t]);
#pragma unroll
        for (int t = 0; t < NB; ++t) d[t] = mma_f16(a_hi1, b[3][t], d[t]);
        fold(d);
      } else {
        u32x4_t a[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          a[j] = LX ? xa[j]
                    : u32x4_t{bf16x2_to_f16x2(xv[j].x), bf16x2_to_f16x2(xv[j].y), bf16x2_to_f16x2(xv[j].z),
                              bf16x2_to_f16x2(xv[j].w)};
        f32x4_t d[NB];
        if constexpr (kGrouped) {
#pragma unroll
          for (int t = 0; t < NB; ++t) d[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int t = 0; t < NB; ++t) {
            const uint32_t w0 = st.c[t][j >> 1][2 * (j & 1)], w1 = st.c[t][j >> 1][2 * (j & 1) + 1];
            const u32x4_t b = {add_f16x2(__builtin_amdgcn_perm(0x64646464u, w0, 0x04010400u), kF16Minus1152),
                               add_f16x2(__builtin_amdgcn_perm(0x64646464u, w0, 0x04030402u), kF16Minus1152),
                               add_f16x2(__builtin_amdgcn_perm(0x64646464u, w1, 0x04010400u), kF16Minus1152),
                               add_f16x2(__builtin_amdgcn_perm(0x64646464u, w1, 0x04030402u), kF16Minus1152)};
            if constexpr (kGrouped) d[t] = mma_f16(a[j], b, d[t]);
            else acc[t] = mma_f16(a[j], b, acc[t]);
          }
        if constexpr (kGrouped) fold(d);
      }
    } else {
      // exact path: bf16 codes (q, or q - z) against bf16 x, one tile at a time
#pragma unroll
      for (int t = 0; t < NB; ++t) {
        f32x4_t dt = {0.f, 0.f, 0.f, 0.f};  // this tile's partial (group-128)
        if constexpr (kW4) {
          const float z = (float)((st.zb[t] >> zshift) & 15u);
          auto ex = [&](uint32_t w, int i) {
            return pack_bf16x2((float)((w >> (4 * i)) & 15u) - z, (float)((w >> (16 + 4 * i)) & 15u) - z);
          };
          const uint32_t w0 = st.c[t][0][0], w1 = st.c[t][0][1], w2 = st.c[t][0][2], w3 = st.c[t][0][3];
          const u32x4_t a_lo0 = {xv[0].x, xv[0].z, xv[1].x, xv[1].z};
          const u32x4_t a_lo1 = {xv[2].x, xv[2].z, xv[3].x, xv[3].z};
          const u32x4_t a_hb0 = {xv[0].y, xv[0].w, xv[1].y, xv[1].w};
          const u32x4_t a_hb1 = {xv[2].y, xv[2].w, xv[3].y, xv[3].w};
          dt = mma_bf16(a_lo0, u32x4_t{ex(w0, 0), ex(w0, 2), ex(w1, 0), ex(w1, 2)}, dt);
          dt = mma_bf16(a_lo1, u32x4_t{ex(w2, 0), ex(w2, 2), ex(w3, 0), ex(w3, 2)}, dt);
          dt = mma_bf16(a_hb0, u32x4_t{ex(w0, 1), ex(w0, 3), ex(w1, 1), ex(w1, 3)}, dt);
          dt = mma_bf16(a_hb1, u32x4_t{ex(w2, 1), ex(w2, 3), ex(w3, 1), ex(w3, 3)}, dt);
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            uint32_t b0, b1, b2, b3;
            i8_word_to_bf16(st.c[t][j >> 1][2 * (j & 1)], b0, b1);
            i8_word_to_bf16(st.c[t][j >> 1][2 * (j & 1) + 1], b2, b3);
            const u32x4_t b = {b0, b1, b2, b3};
            const u32x4_t a = {xv[j].x, xv[j].y, xv[j].z, xv[j].w};
            if constexpr (kGrouped) dt = mma_bf16(a, b, dt);
            else acc[t] = mma_bf16(a, b, acc[t]);
          }
        }
        if constexpr (kGrouped) fold1(t, dt);
      }
    }
  };

  // A wave's units u0 + wave, + W, ...  Without LX each unit loads and multiplies in
  // turn (a second operand set, x included, halves the resident waves: measured slower
  // on MI355X).  With LX the set holds codes and metadata only, and the next unit's
  // loads go out before the current unit's products (unconditionally inside the paired
  // loop, so that waiting for one set never drains the other).
  if constexpr (!LX) {
    for (int u = u0 + wu; u < u1; u += W) {
      Set st;
      load(st, u);
      compute(st, u);
    }
  } else {
    // two operand sets: the next unit's loads go out before the current unit's
    // products (unconditionally inside the paired loop, so that waiting for one set
    // never drains the other); the first unit's loads went out before the x prologue
    if (n_my > 0) {
      int u = first, i = 0;
      for (; i + 2 < n_my; i += 2, u += 2 * W) {
        load(sb, u + W);
        compute(sa, u);
        load(sa, u + 2 * W);
        compute(sb, u + W);
      }
      if (i + 1 < n_my) {
        load(sb, u + W);
        compute(sa, u);
        compute(sb, u + W);
      } else {
        compute(sa, u);
      }
    }
  }
  // the waves' partial sums meet in LDS and are added in wave order
#pragma unroll
  for (int t = 0; t < NB; ++t)
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int m = 4 * (int)lk + i;
      if (m < Mr) red[wave][t][m][ln] = acc[t][i];
    }
  __syncthreads();
  for (int o = threadIdx.x; o < NB * Mr * 16; o += blockDim.x) {
    const int t = o / (Mr * 16), m = (o / 16) % Mr, n = 16 * (tile0 + t) + (o & 15);
    if (tile0 + t >= T16 || n >= N) continue;
    float v = 0.f;
    for (int w = 0; w < W; ++w) v += red[w][t][m][o & 15];
    if (S == 1)
      y[(size_t)m * N + n] = f32_to_bf16(with_res<false>(kGrouped ? v : bf16_to_f32(scales[n]) * v, res,
                                                         (size_t)m * N + n));
    else part[((size_t)s * Mr + m) * N + n] = v;
  }
}

template <int FMT, int M, int NB>
void launch_mma_nb(dim3 grid, dim3 block, const uint8_t* qw, const uint16_t* sc, const uint8_t* zs,
                   const uint16_t* x, uint16_t* y, const uint16_t* res, float* part, int K, int N, int Mt, hipStream_t st) {
  // x in LDS when the largest split range's fp16 x fits (ranges differ by one unit at most)
  const int U = (K + kGroup - 1) / kGroup, S = (int)grid.y;
  const int lx = lx_bytes(Mt, (U + S - 1) / S);
  if (lx <= kLxMaxBytes)
    gemv_mma_kernel<FMT, M, NB, true><<<grid, block, lx, st>>>(qw, sc, zs, x, y, part, K, N, Mt, res);
  else
    gemv_mma_kernel<FMT, M, NB, false><<<grid, block, 0, st>>>(qw, sc, zs, x, y, part, K, N, Mt, res);
}

template <int FMT, int M>
void launch_mma(int nb, dim3 grid, dim3 block, const uint8_t* qw, const uint16_t* sc, const uint8_t* zs,
                const uint16_t* x, uint16_t* y, const uint16_t* res, float* part, int K, int N, int Mt, hipStream_t st) {
  switch (nb) {
    case 1: launch_mma_nb<FMT, M, 1>(grid, block, qw, sc, zs, x, y, res, part, K, N, Mt, st); break;
    case 2: launch_mma_nb<FMT, M, 2>(grid, block, qw, sc, zs, x, y, res, part, K, N, Mt, st); break;
    default: launch_mma_nb<FMT, M, 4>(grid, block, qw, sc, zs, x, y, res, part, K, N, Mt, st); break;
  }
}

template <int FMT, int M, int RR>
void launch_rr(bool pf, bool xf, dim3 grid, dim3 block, const uint8_t* qw, const uint16_t* sc, const uint8_t* zs,
               const uint16_t* x, uint16_t* y, const uint16_t* res, float* part, int K, int N, int gshift, hipStream_t st) {
  if (xf) {  // fp16 activations: no prefetch variant (the launcher checks)
    gemv_kernel<FMT, M, RR, false, true><<<grid, block, 0, st>>>(qw, sc, zs, x, y, part, K, N, gshift, res);
    return;
  }
  if constexpr (prefetch_allowed(FMT, RR, M)) {
    if (pf) {
      gemv_kernel<FMT, M, RR, true><<<grid, block, 0, st>>>(qw, sc, zs, x, y, part, K, N, gshift, res);
      return;
    }
  }
  gemv_kernel<FMT, M, RR, false><<<grid, block, 0, st>>>(qw, sc, zs, x, y, part, K, N, gshift, res);
}

// rows: 4, 8 or 16, optionally | kGemvPrefetch (checked by the caller)
template <int FMT, int M>
wq_status launch_m(int rows, bool xf, dim3 grid, dim3 block, const uint8_t* qw, const uint16_t* sc,
                   const uint8_t* zs, const uint16_t* x, uint16_t* y, const uint16_t* res, float* part, int K, int N,
                   int gshift, hipStream_t st) {
  const bool pf = (rows & kGemvPrefetch) != 0;
  switch (rows & ~kGemvPrefetch) {
    case 4: launch_rr<FMT, M, 4>(pf, xf, grid, block, qw, sc, zs, x, y, res, part, K, N, gshift, st); break;
    case 8: launch_rr<FMT, M, 8>(pf, xf, grid, block, qw, sc, zs, x, y, res, part, K, N, gshift, st); break;
    case 16: launch_rr<FMT, M, 16>(pf, xf, grid, block, qw, sc, zs, x, y, res, part, K, N, gshift, st); break;
    default: return fail(WQ_ERR_INVALID_ARG, "wq_gemv: rows per wave must be 4, 8 or 16");
  }
  return WQ_OK;
}

template <int FMT>
wq_status launch_fmt(const wq_weight* w, const uint16_t* x, int M, uint16_t* y, int split_k,
                     int waves, int rows, void* ws, bool xf, const uint16_t* res, hipStream_t st) {
  const int K = (int)w->K, N = (int)w->N;
  if (xf && (rows & (kGemvMfma | kGemvPrefetch)))
    return fail(WQ_ERR_UNSUPPORTED, "wq_gemv: fp16 activations take the dot2 GEMV without prefetch");
  const int gshift = meta_group(w->fmt) == 32 ? 5 : meta_group(w->fmt) == 64 ? 6 : 7;
  float* part = (float*)ws;
  const uint8_t* qw = (const uint8_t*)w->qweight;
  const uint16_t* sc = (const uint16_t*)w->scales;
  const uint8_t* zs = (const uint8_t*)w->zeros;
  wq_status r = WQ_OK;
  if (rows & kGemvMfma) {
    const int nb = (rows & 0xFF) / R;
    dim3 grid((unsigned)((row_tiles(N) + nb - 1) / nb), split_k);
    dim3 block(64 * waves);
    switch (M) {
      case 1: launch_mma<FMT, 1>(nb, grid, block, qw, sc, zs, x, y, res, part, K, N, 1, st); break;
      case 2: launch_mma<FMT, 2>(nb, grid, block, qw, sc, zs, x, y, res, part, K, N, 2, st); break;
      case 3: launch_mma<FMT, 3>(nb, grid, block, qw, sc, zs, x, y, res, part, K, N, 3, st); break;
      case 4: launch_mma<FMT, 4>(nb, grid, block, qw, sc, zs, x, y, res, part, K, N, 4, st); break;
      case 5: launch_mma<FMT, 5>(nb, grid, block, qw, sc, zs, x, y, res, part, K, N, 5, st); break;
      case 6: launch_mma<FMT, 6>(nb, grid, block, qw, sc, zs, x, y, res, part, K, N, 6, st); break;
      case 7: launch_mma<FMT, 7>(nb, grid, block, qw, sc, zs, x, y, res, part, K, N, 7, st); break;
      default:
        if (M > kMmaTokens) return fail(WQ_ERR_INVALID_ARG, "matrix-core GEMV: M must be in 1..16");
        launch_mma<FMT, kMmaTokens>(nb, grid, block, qw, sc, zs, x, y, res, part, K, N, M, st);
        break;
    }
  } else {
  dim3 grid((unsigned)(row_tiles(N) * (R / (rows & ~kGemvPrefetch))), split_k);
  dim3 block(64 * waves);
  switch (M) {
    case 1: r = launch_m<FMT, 1>(rows, xf, grid, block, qw, sc, zs, x, y, res, part, K, N, gshift, st); break;
    case 2: r = launch_m<FMT, 2>(rows, xf, grid, block, qw, sc, zs, x, y, res, part, K, N, gshift, st); break;
    case 3: r = launch_m<FMT, 3>(rows, xf, grid, block, qw, sc, zs, x, y, res, part, K, N, gshift, st); break;
    case 4: r = launch_m<FMT, 4>(rows, xf, grid, block, qw, sc, zs, x, y, res, part, K, N, gshift, st); break;
    case 5: r = launch_m<FMT, 5>(rows, xf, grid, block, qw, sc, zs, x, y, res, part, K, N, gshift, st); break;
    case 6: r = launch_m<FMT, 6>(rows, xf, grid, block, qw, sc, zs, x, y, res, part, K, N, gshift, st); break;
    case 7: r = launch_m<FMT, 7>(rows, xf, grid, block, qw, sc, zs, x, y, res, part, K, N, gshift, st); break;
    default: return fail(WQ_ERR_INVALID_ARG, "wq_gemv: M must be in 1..7");
  }
  }
  if (r != WQ_OK) return r;
  WQ_HIP_CHECK(hipGetLastError());
  if (split_k > 1) {
    const int64_t MN = (int64_t)M * N;
    if (xf) splitk_reduce_kernel<FMT, true><<<(unsigned)((MN + 255) / 256), 256, 0, st>>>(part, sc, y, M, N, split_k, res);
    else splitk_reduce_kernel<FMT><<<(unsigned)((MN + 255) / 256), 256, 0, st>>>(part, sc, y, M, N, split_k, res);
    WQ_HIP_CHECK(hipGetLastError());
  }
  return WQ_OK;
}

}  // namespace

size_t gemv_workspace_bytes(int64_t N, int64_t M, int split_k) {
  if (split_k <= 1) return 0;
  return (size_t)split_k * (size_t)M * (size_t)N * sizeof(float);
}

int gemv_max_waves(int fmt, int M, int rows) {
  if (rows & kGemvMfma) {
    const int rr = rows & ~kGemvMfma;
    if (M < 1 || M > kMmaTokens || small_group(fmt)) return 0;
    return (rr == 16 || rr == 32 || rr == 64) ? kMmaMaxWaves : 0;
  }
  const int rr = rows & ~kGemvPrefetch;
  const bool pf = (rows & kGemvPrefetch) != 0;
  fmt = family(fmt);
  if (rr != 4 && rr != 8 && rr != 16) return 0;
  if (pf && !prefetch_allowed(fmt, rr, M)) return 0;
  return max_waves_r(fmt, rr, M, pf);
}

int64_t gemv_slices(int64_t K, int fmt) {
  const int64_t slice = 64 * (is_w4(fmt) ? 32 : 16);
  return (K + slice - 1) / slice;
}

int gemv_default_rows(int64_t K, int64_t N, int fmt, int M) {
  // thin waves (4 rows) keep many waves resident when the matrix is small; more
  // rows per wave share each x chunk (and its conversion) among more rows, which
  // pays when there are many row tiles or several tokens (measured on MI355X)
  (void)K;
  if (is_w4(fmt) && M >= 5) return 8;  // 16 rows x 5+ tokens of uint4 spill registers
  if (M >= 4) return N >= 16384 ? 16 : 8;
  if (is_w4(fmt)) return 8;
  return N >= 16384 ? 8 : 4;
}

int gemv_default_waves(int64_t K, int64_t N, int fmt, int M, int split_k, int rows) {
  if (rows & kGemvMfma) {
    // about four 128-k units per wave
    const int64_t groups = ((K + kGroup - 1) / kGroup + split_k - 1) / split_k;
    const int64_t wv = (groups + 3) / 4;
    return (int)(wv < 1 ? 1 : (wv > kMmaMaxWaves ? kMmaMaxWaves : wv));
  }
  // one K slice per wave, as many waves as the register budget allows
  const int64_t per_split = (gemv_slices(K, fmt) + split_k - 1) / split_k;
  (void)N;
  const int cap = gemv_max_waves(fmt, M, rows);
  return (int)(per_split < cap ? (per_split < 1 ? 1 : per_split) : cap);
}

wq_status launch_gemv(const wq_weight* w, const uint16_t* x, int M, uint16_t* y, int split_k,
                      int waves, int rows, void* ws, hipStream_t s, bool xf, const uint16_t* res) {
  const int cap = gemv_max_waves(w->fmt, M, rows);
  if (cap == 0) return fail(WQ_ERR_INVALID_ARG, "wq_gemv: rows per wave must be 4, 8 or 16");
  if (waves < 1 || waves > cap)
    return fail(WQ_ERR_UNSUPPORTED, "wq_gemv: at this M and rows a workgroup holds 1.." +
                                        std::to_string(cap) + " waves");
  if (w->fmt == WQ_FMT_W4_PC) return fail(WQ_ERR_UNSUPPORTED, "wq_gemv: per-channel W4 runs through its compute view");
  switch (family(w->fmt)) {
    case WQ_FMT_W8_PC: return launch_fmt<WQ_FMT_W8_PC>(w, x, M, y, split_k, waves, rows, ws, xf, res, s);
    case WQ_FMT_W8_G128: return launch_fmt<WQ_FMT_W8_G128>(w, x, M, y, split_k, waves, rows, ws, xf, res, s);
    case WQ_FMT_W4_G128: return launch_fmt<WQ_FMT_W4_G128>(w, x, M, y, split_k, waves, rows, ws, xf, res, s);
  }
  return fail(WQ_ERR_UNSUPPORTED, "wq_gemv: unknown format");
}

}  // namespace wq
