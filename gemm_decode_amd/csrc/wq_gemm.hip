// Prefill GEMM: y[M][N] = x[M][K] . dequant(W)[N][K]^T for M >= 8 tokens.
//
// The tileInfer README ("Key Optimizations") runs prefill as a bf16 GEMM whose
// int8 weights are dequantized to bf16 on the fly; the Marlin benchmark page
// (intro) attributes its large-M gains to keeping accumulators out of spills and
// sizing shared memory to the tile.  This kernel is the gfx950 form of that step:
//
//   * a 256-thread workgroup computes a BM x BN tile of y; its four waves (2 x 2)
//     each own a 64 x 64 sub-tile made of 2 x 2 v_mfma_f32_32x32x16_bf16 blocks;
//   * per K step (BK = 64) the bf16 x tile is copied to LDS and the packed codes
//     are converted to EXACT bf16 values (int8 q, or q - z for uint4, both exact
//     in bf16) on their way into LDS; scales are never folded into the bf16
//     operand, because rounding q*s to bf16 loses accuracy;
//   * the next K step's global loads are in flight while the MFMAs of the current
//     step run (register prefetch, single LDS buffer);
//   * per-channel W8 multiplies by s[n] in the epilogue; group-128 formats keep a
//     second fp32 accumulator that is scaled by s[n][g] and folded in at the end
//     of every 128-element group.
#include "wq_internal.h"
#include <algorithm>
#include <type_traits>
#include <atomic>

namespace wq {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 h16x2_t __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDA = BK + 8;  // LDS row pitch in bf16 (16-byte pad)

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v;
  v.x = (__bf16)lo;
  v.y = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ float f16_to_f32(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }
// two small integers (exact in both 16-bit types) as a pair of the operand type: bf16,
// or fp16 for fp16 activations (XF)
template <bool XF>
__device__ __forceinline__ uint32_t pack_x2(float lo, float hi) {
  if constexpr (XF) return __builtin_bit_cast(uint32_t, h16x2_t{(_Float16)lo, (_Float16)hi});
  else return pack_bf16x2(lo, hi);
}
// an fp32 result as the output type (nearest even): bf16, or fp16 with XF
template <bool XF>
__device__ __forceinline__ uint16_t f32_to_out(float v) {
  if constexpr (XF) return __builtin_bit_cast(uint16_t, (_Float16)v);
  else return __builtin_bit_cast(uint16_t, (__bf16)v);
}
// the fp32 result plus element i of the residual (y's type, widened exactly) when there
// is one, so that y is rounded once; the residual may be y itself (each element is read
// by the thread that writes it, before the write)
template <bool XF>
__device__ __forceinline__ float with_res(float v, const uint16_t* res, size_t i) {
  if (!res) return v;
  return v + (XF ? f16_to_f32(res[i]) : bf16_to_f32(res[i]));
}

// gfx950 int8 codes are u = q + 128; flipping the sign bit gives q (as bf16, or fp16 with XF).
template <bool XF = false>
__device__ __forceinline__ uint4 i8x16_to_bf16_lo(uint4 v) {
  auto cvt = [](uint32_t d) -> uint2 {
    d ^= 0x80808080u;
    return make_uint2(pack_x2<XF>((float)(int8_t)(d & 0xFFu), (float)(int8_t)((d >> 8) & 0xFFu)),
                      pack_x2<XF>((float)(int8_t)((d >> 16) & 0xFFu), (float)(int8_t)(d >> 24)));
  };
  uint2 a = cvt(v.x), b = cvt(v.y);
  return make_uint4(a.x, a.y, b.x, b.y);
}
template <bool XF = false>
__device__ __forceinline__ uint4 i8x16_to_bf16_hi(uint4 v) {
  return i8x16_to_bf16_lo<XF>(make_uint4(v.z, v.w, 0, 0));
}

// One gfx950-layout W4 word (8 codes, nibbles q0 q2 q4 q6 q1 q3 q5 q7) -> 8 exact bf16 (q - z)
// (fp16 with XF).
template <bool XF = false>
__device__ __forceinline__ uint4 w4_word_to_bf16(uint32_t w, float z) {
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = (float)((w >> (4 * i)) & 0xFu) - z;
    const float hi = (float)((w >> (16 + 4 * i)) & 0xFu) - z;
    o[i] = pack_x2<XF>(lo, hi);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// gshift: the grouped formats' group size is 2^gshift k (32, 64 or 128).  XF: x and y in
// fp16 (fp16 activations): the codes go to LDS as fp16 and the products run on
// v_mfma_f32_32x32x16_f16 (every code value and every fp16 x is exact in fp16, their
// products in fp32).
template <int FMT, bool XF = false>
__global__ __launch_bounds__(256) void gemm_kernel(const uint8_t* __restrict__ qw,
                                                     const uint16_t* __restrict__ scales,
                                                     const uint8_t* __restrict__ zeros,
                                                     const uint16_t* __restrict__ x,
                                                     uint16_t* y, int M, int K, int N, int gshift,
                                                     const uint16_t* res) {
  __shared__ __attribute__((aligned(16))) uint16_t As[BM * LDA];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[BN * LDA];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
  const int G = K >> gshift, gmask = (1 << gshift) - 1;
  constexpr bool kGrouped = FMT != WQ_FMT_W8_PC;

  // ---- global -> register staging
  uint4 xa[4];
  uint4 wb[2];
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = tid + 256 * j;
      const int row = i >> 3, col = (i & 7) * 8;
      const int m = m0 + row, k = k0 + col;
      xa[j] = (m < M && k < K) ? *reinterpret_cast<const uint4*>(x + (size_t)m * K + k)
                               : make_uint4(0, 0, 0, 0);
    }
    if constexpr (FMT != WQ_FMT_W4_G128) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int i = tid + 256 * j;
        const int row = i >> 2, col = (i & 3) * 16;
        const int n = min(n0 + row, N - 1), k = k0 + col;
        wb[j] = (k < K) ? *reinterpret_cast<const uint4*>(qw + tiled_offset(n, k, N, K)) : make_uint4(0, 0, 0, 0);
      }
    } else {
      const int row = tid >> 1, col = (tid & 1) * 32;
      const int n = min(n0 + row, N - 1);
      wb[0] = *reinterpret_cast<const uint4*>(qw + tiled_offset(n, (k0 + col) / 2, N, K / 2));
    }
  };
  auto store_tile = [&](int k0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = tid + 256 * j;
      const int row = i >> 3, col = (i & 7) * 8;
      *reinterpret_cast<uint4*>(&As[row * LDA + col]) = xa[j];
    }
    if constexpr (FMT != WQ_FMT_W4_G128) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int i = tid + 256 * j;
        const int row = i >> 2, col = (i & 3) * 16;
        *reinterpret_cast<uint4*>(&Bs[row * LDA + col]) = i8x16_to_bf16_lo<XF>(wb[j]);
        *reinterpret_cast<uint4*>(&Bs[row * LDA + col + 8]) = i8x16_to_bf16_hi<XF>(wb[j]);
      }
    } else {
      const int row = tid >> 1, col = (tid & 1) * 32;
      const int n = min(n0 + row, N - 1);
      const int g = (k0 + col) >> gshift;  // this thread's 32 k lie in one group
      const uint32_t zb = zeros[(((size_t)(n / kGemvTileRows) * G + g) * kGemvTileRows + n % kGemvTileRows) / 2];
      const float z = (float)((zb >> ((n & 1) * 4)) & 0xFu);
      *reinterpret_cast<uint4*>(&Bs[row * LDA + col + 0]) = w4_word_to_bf16<XF>(wb[0].x, z);
      *reinterpret_cast<uint4*>(&Bs[row * LDA + col + 8]) = w4_word_to_bf16<XF>(wb[0].y, z);
      *reinterpret_cast<uint4*>(&Bs[row * LDA + col + 16]) = w4_word_to_bf16<XF>(wb[0].z, z);
      *reinterpret_cast<uint4*>(&Bs[row * LDA + col + 24]) = w4_word_to_bf16<XF>(wb[0].w, z);
    }
  };

  floatx16 acc[2][2], tmp[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int a = 0; a < 16; ++a) acc[i][j][a] = tmp[i][j][a] = 0.f;

  const int l32 = lane & 31, lh = lane >> 5;
  load_tile(0);
  for (int k0 = 0; k0 < K; k0 += BK) {
    __syncthreads();
    store_tile(k0);
    __syncthreads();
    if (k0 + BK < K) load_tile(k0 + BK);
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      bf16x8_t af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = wm * 64 + i * 32 + l32;
        af[i] = *reinterpret_cast<const bf16x8_t*>(&As[row * LDA + kk + 8 * lh]);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int row = wn * 64 + j * 32 + l32;
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(&Bs[row * LDA + kk + 8 * lh]);
      }
      auto mfma = [&](const bf16x8_t& a, const bf16x8_t& b, const floatx16& c) -> floatx16 {
        if constexpr (XF)
          return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(h16x8_t, a), __builtin_bit_cast(h16x8_t, b),
                                                        c, 0, 0, 0);
        else
          return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
      };
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          if constexpr (kGrouped)
            tmp[i][j] = mfma(af[i], bfr[j], tmp[i][j]);
          else
            acc[i][j] = mfma(af[i], bfr[j], acc[i][j]);
        }
      // the end of a group: its partial sums, times the group scale, into acc
      if constexpr (kGrouped) {
        if (((k0 + kk + 16) & gmask) == 0) {
          const int g = (k0 + kk) >> gshift;
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int n = min(n0 + wn * 64 + j * 32 + l32, N - 1);
            const uint16_t sb = scales[((size_t)(n / kGemvTileRows) * G + g) * kGemvTileRows + n % kGemvTileRows];
            const float s = (FMT == WQ_FMT_W8_G128) ? bf16_to_f32(sb) : f16_to_f32(sb);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
              for (int a = 0; a < 16; ++a) {
                acc[i][j][a] = fmaf(s, tmp[i][j][a], acc[i][j][a]);
                tmp[i][j][a] = 0.f;
              }
          }
        }
      }
    }
  }

  // ---- epilogue: D[row = 8*(a/4) + 4*(lane/32) + a%4][col = lane%32] of each 32x32 block
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = n0 + wn * 64 + j * 32 + l32;
    if (n >= N) continue;
    const float s = (FMT == WQ_FMT_W8_PC) ? bf16_to_f32(scales[n]) : 1.f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int a = 0; a < 16; ++a) {
        const int m = m0 + wm * 64 + i * 32 + 8 * (a >> 2) + 4 * lh + (a & 3);
        if (m < M) y[(size_t)m * N + n] = f32_to_out<XF>(with_res<XF>(s * acc[i][j][a], res, (size_t)m * N + n));
      }
  }
}

// ---------------------------------------------------------------------------------
// Large-M kernel: 4 waves (2 x 2).  Per-channel W8: 256 x 256 workgroup tile, each wave
// 128 x 128 = a 4 x 4 grid of 32 x 32 MFMA blocks (256 fp32 accumulators per lane).
// Wave tiles this large halve the LDS operand traffic per MFMA compared with 64 x 64
// tiles, which would otherwise keep LDS as busy as the matrix cores.  Group-128
// formats keep a second accumulator for the current group (its fp32 partial is
// scaled by s[n][g] and added at the end of the group), so their wave tile is
// 128 x 64 (256 x 128 per workgroup).  Two LDS stages (x tile and exact-bf16 weight
// tile): while the MFMAs read one, the next K step is loaded from memory, converted
// and written into the other; one barrier per step.
//
// Workgroups are numbered so that XCD x (workgroup ids x, x + 8, ...) runs a
// contiguous range of column blocks, each for every row block in turn: a weight
// strip is fetched into that XCD's L2 once and reused by all row blocks.
constexpr int BM2 = 256, BK2 = 64;
constexpr int P2 = BK2 + 8;                  // LDS row pitch in bf16 (16-byte pad)

template <int FMT>
struct Big {
  static constexpr bool kGrouped = FMT != WQ_FMT_W8_PC;
  static constexpr int JN = kGrouped ? 2 : 4;  // 32-wide column blocks per wave
  static constexpr int BN = 64 * JN;           // columns per workgroup
  static constexpr int STAGE = (BM2 + BN) * P2;
};

template <int FMT>
__global__ __launch_bounds__(256, 1) void gemm_big_kernel(const uint8_t* __restrict__ qw,
                                                           const uint16_t* __restrict__ scales,
                                                           const uint8_t* __restrict__ zeros,
                                                           const uint16_t* __restrict__ x,
                                                           uint16_t* y, int M, int K, int N,
                                                           const uint16_t* res) {
  using B_ = Big<FMT>;
  constexpr int JN = B_::JN, BN2 = B_::BN, STAGE2 = B_::STAGE;
  constexpr bool kW4 = FMT == WQ_FMT_W4_G128;
  constexpr bool kGrouped = B_::kGrouped;
  constexpr int TPR = 256 / BN2;                 // threads staging one weight row
  constexpr int WCH = (kW4 ? 2 : 4) / TPR;      // 16-byte code chunks per thread and K step
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * STAGE2];

  // ---- XCD-aware tile order
  const int mblocks = (M + BM2 - 1) / BM2, nblocks = (N + BN2 - 1) / BN2;
  const int total = mblocks * nblocks;
  const int per_xcd = (total + 7) / 8;
  const int lin = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (lin >= total) return;
  const int nb = lin / mblocks, mb = lin % mblocks;
  const int n0 = nb * BN2, m0 = mb * BM2;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, lh = lane >> 5;
  const int G = K / kGroup;
  const int64_t row_bytes = kW4 ? K / 2 : K;
  const int brow = tid / TPR, bpart = tid % TPR;  // weight row and part this thread stages
  const int nrow = min(n0 + brow, N - 1);

  uint4 xr[8], wr[WCH];
  auto load_global = [&](int k0) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int c = tid + 256 * j, row = c >> 3, col = (c & 7) * 8;
      const int m = m0 + row, k = k0 + col;
      xr[j] = (m < M && k < K) ? *reinterpret_cast<const uint4*>(x + (size_t)m * K + k) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < WCH; ++j) {
      const int b = (kW4 ? k0 / 2 : k0) + 16 * (bpart * WCH + j);  // byte of the packed row
      wr[j] = b < row_bytes ? *reinterpret_cast<const uint4*>(qw + tiled_offset(nrow, b, N, row_bytes))
                            : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_lds = [&](int st, int k0) {
    uint16_t* A = lds + st * STAGE2;
    uint16_t* Bt = A + BM2 * P2;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int c = tid + 256 * j, row = c >> 3, col = (c & 7) * 8;
      *reinterpret_cast<uint4*>(&A[row * P2 + col]) = xr[j];
    }
    uint16_t* Brow = Bt + brow * P2;
    if constexpr (!kW4) {
#pragma unroll
      for (int j = 0; j < WCH; ++j) {
        const int kc = 16 * (bpart * WCH + j);
        *reinterpret_cast<uint4*>(&Brow[kc]) = i8x16_to_bf16_lo(wr[j]);
        *reinterpret_cast<uint4*>(&Brow[kc + 8]) = i8x16_to_bf16_hi(wr[j]);
      }
    } else {
      const int g = k0 / kGroup;
      const uint8_t zb = zeros[(((size_t)(nrow / kGemvTileRows) * G + g) * kGemvTileRows + nrow % kGemvTileRows) / 2];
      const float z = (float)((zb >> ((nrow & 1) * 4)) & 0xFu);
#pragma unroll
      for (int j = 0; j < WCH; ++j) {
        const int kc = 32 * (bpart * WCH + j);
        *reinterpret_cast<uint4*>(&Brow[kc + 0]) = w4_word_to_bf16(wr[j].x, z);
        *reinterpret_cast<uint4*>(&Brow[kc + 8]) = w4_word_to_bf16(wr[j].y, z);
        *reinterpret_cast<uint4*>(&Brow[kc + 16]) = w4_word_to_bf16(wr[j].z, z);
        *reinterpret_cast<uint4*>(&Brow[kc + 24]) = w4_word_to_bf16(wr[j].w, z);
      }
    }
  };

  int ncol[JN];
#pragma unroll
  for (int j = 0; j < JN; ++j) ncol[j] = min(n0 + wn * (32 * JN) + j * 32 + l32, N - 1);
  auto gscale = [&](int n, int g) -> float {
    const uint16_t sb = scales[((size_t)(n / kGemvTileRows) * G + g) * kGemvTileRows + n % kGemvTileRows];
    return (FMT == WQ_FMT_W8_G128) ? bf16_to_f32(sb) : f16_to_f32(sb);
  };

  floatx16 acc[4][JN], tmp[4][JN];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < JN; ++j)
#pragma unroll
      for (int a = 0; a < 16; ++a) acc[i][j][a] = tmp[i][j][a] = 0.f;

  const int KS = (K + BK2 - 1) / BK2;
  load_global(0);
  store_lds(0, 0);
  __syncthreads();
  for (int ks = 0; ks < KS; ++ks) {
    const int k0 = ks * BK2;
    if (ks + 1 < KS) load_global(k0 + BK2);
    const uint16_t* A = lds + (ks & 1) * STAGE2;
    const uint16_t* Bt = A + BM2 * P2;
#pragma unroll
    for (int kk = 0; kk < BK2; kk += 16) {
      bf16x8_t af[4], bfr[JN];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t*>(&A[(wm * 128 + i * 32 + l32) * P2 + kk + 8 * lh]);
#pragma unroll
      for (int j = 0; j < JN; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(&Bt[(wn * (32 * JN) + j * 32 + l32) * P2 + kk + 8 * lh]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < JN; ++j) {
          if constexpr (kGrouped)
            tmp[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], tmp[i][j], 0, 0, 0);
          else
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
    }
    if constexpr (kGrouped) {
      if ((k0 + BK2) % kGroup == 0) {
        const int g = k0 / kGroup;
#pragma unroll
        for (int j = 0; j < JN; ++j) {
          const float sc = gscale(ncol[j], g);
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int a = 0; a < 16; ++a) {
              acc[i][j][a] = fmaf(sc, tmp[i][j][a], acc[i][j][a]);
              tmp[i][j][a] = 0.f;
            }
        }
      }
    }
    if (ks + 1 < KS) store_lds((ks + 1) & 1, k0 + BK2);
    __syncthreads();
  }

  // ---- epilogue: D[row = 8*(a/4) + 4*(lane/32) + a%4][col = lane%32] of each 32x32 block
#pragma unroll
  for (int j = 0; j < JN; ++j) {
    const int n = n0 + wn * (32 * JN) + j * 32 + l32;
    const float sc = kGrouped ? 1.f : bf16_to_f32(scales[ncol[j]]);
    if (n >= N) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int a = 0; a < 16; ++a) {
        const int m = m0 + wm * 128 + i * 32 + 8 * (a >> 2) + 4 * lh + (a & 3);
        if (m < M) y[(size_t)m * N + n] = f32_to_out<false>(with_res<false>(sc * acc[i][j][a], res, (size_t)m * N + n));
      }
  }
}

// ---------------------------------------------------------------------------------
// Per-channel W8, large M: operands travel global -> LDS by LDS-DMA
// (global_load_lds_dwordx4), so no register staging, and three LDS stages let each
// K step's loads be issued two steps before use.  The 256 x 256 workgroup tile is
// split over 4 waves of 128 x 128 (4 x 4 blocks of v_mfma_f32_32x32x16_bf16).
//
// LDS stage (48 KB): x tile [256 rows][64 k] bf16 as 128-byte rows, then codes
// [256 rows][64 k] int8 as 64-byte rows.  A DMA instruction writes 64 lanes x 16 bytes
// to 1 KB of consecutive LDS, so bank conflicts are avoided by choosing which 16-byte
// chunk each lane fetches: chunk c of x row r sits at position c ^ fx(r), chunk c of
// code row n at position c ^ fw(n).  Both swizzles keep any 8 (and any 16) rows that
// one ds_read_b128 phase touches on distinct banks.
//
// K order inside a 32-wide slice: lane half h of MFMA s (0 or 1) takes k = 16h + 8s +
// 0..7, so one 16-byte code chunk (16 k) feeds both MFMAs of a lane half.  The same
// permutation is applied to x, so every product pairs equal k.
//
// Per step t: MFMAs of slice 0 while slice 1's fragments are read and its codes
// converted to exact bf16 (q = u - 128); wait for this wave's DMA of step t + 1,
// barrier; issue the DMA of step t + 3 into the stage just finished (so each DMA has
// two steps to land); MFMAs of slice 1 while slice 0 of step t + 1 is read.
constexpr int DBM = 256, DBN = 256, DBK = 64;
constexpr int DA_BYTES = DBM * DBK * 2, DB_BYTES = DBN * DBK, DSTAGE = DA_BYTES + DB_BYTES;

__device__ __forceinline__ int swz_x(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int swz_w(int n) { return ((n >> 2) ^ (((n >> 1) & 1) << 1)) & 3; }

// One LDS-DMA instruction: lane i copies 16 bytes from g (its own address) to LDS
// byte l + 16 i (l is wave-uniform).  It is written out rather than taken from
// __builtin_amdgcn_global_load_lds because the compiler cannot tell the three stages
// apart and would drain every DMA in flight (vmcnt(0)) before each LDS read; the
// kernel instead waits explicitly, and only for the step it is about to read.  The
// instruction writes no register.
__device__ __forceinline__ void dma16(const void* g, uint8_t* l) {
  // The low 32 bits of a generic pointer into the LDS aperture are the LDS address.
  const uint32_t la = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)l);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(la), "v"(g) : "memory", "m0");
}

// Which 256 x 256 output tile and which K range a workgroup of the LDS-DMA kernels
// takes, and where its fp32 partials go.  Blocks 0 .. 8 ceil(tail0 / 8) - 1 take
// tiles 0 .. tail0 - 1 (whole, or split over gridDim.y), spread XCD by XCD (block b
// runs on XCD b % 8, which gets a contiguous run of tiles: neighbouring tiles share
// x rows or weight columns in its L2).  The blocks after them take the tiles from
// tail0 on in tailS K ranges each -- a last round of tiles that would leave CUs idle
// -- also XCD by XCD.  Partials: [S][M][N] for the gridDim.y split; for a split tail
// tile its own [tailS][256][256] block, tile by tile from tail0.
struct DmaWork {
  int lin, S, sp;     // tile (XCD-aware linear index), K ranges of the tile, this range
  size_t poff;        // partials of this range: part[poff + (m - pm0) * ppitch + n - pn0]
  int ppitch, pm0, pn0;
};
__device__ __forceinline__ bool dma_work(int M, int N, int tail0, int tailS, DmaWork& w, int tm = DBM) {
  const int mblocks = (M + tm - 1) / tm, nblocks = (N + DBN - 1) / DBN, total = mblocks * nblocks;
  const int b = blockIdx.x, per_full = (tail0 + 7) / 8;
  if (b < 8 * per_full) {
    w.lin = (b & 7) * per_full + (b >> 3);
    if (w.lin >= tail0) return false;
    w.S = gridDim.y;
    w.sp = blockIdx.y;
    w.poff = (size_t)w.sp * M * N;
    w.ppitch = N;
    w.pm0 = w.pn0 = 0;
  } else {
    const int u = b - 8 * per_full, nu = tailS * (total - tail0), per_xcd = (nu + 7) / 8;
    const int lu = (u & 7) * per_xcd + (u >> 3);
    if (lu >= nu) return false;
    w.lin = tail0 + lu / tailS;
    w.S = tailS;
    w.sp = lu % tailS;
    w.poff = (size_t)lu * tm * DBN;  // [tile - tail0][sp] blocks
    w.ppitch = DBN;
    w.pm0 = (w.lin % mblocks) * tm;
    w.pn0 = (w.lin / mblocks) * DBN;
  }
  return true;
}

// WM x WN waves (2 x 2 or 1 x 4) over the 256 x 256 tile: each wave owns RB = 8 / WM
// row blocks and CB = 8 / WN column blocks of 32.  With 1 x 4 every code chunk is
// converted by exactly one wave (half the conversion work of 2 x 2) at the price of
// every wave reading the whole x tile from LDS.
// XF: fp16 activations -- x arrives as fp16 (the same DMA), the codes become exact fp16
// instead of bf16, the products run on v_mfma_f32_32x32x16_f16 and y is fp16.
template <int WM, int WN, int TM, bool XF = false>
__device__ __forceinline__ void dma_w8pc_body(const uint8_t* __restrict__ qw,
                                                                         const uint16_t* __restrict__ scales,
                                                                         const uint16_t* __restrict__ x,
                                                                         uint16_t* y,
                                                                         float* __restrict__ part, int M, int K,
                                                                         int N, int tail0,
                                                                         int tailS, const uint16_t* res) {
  // TM: rows of x per workgroup tile (256, or 64 for a few tokens, where the tile
  // streams the same weights with a quarter of the x traffic and MFMA work)
  constexpr int NW = WM * WN, RB = TM / 32 / WM, CB = 8 / WN;
  constexpr int XI = TM / 8 / NW, WI = 16 / NW;  // x and code DMA instructions per wave and step
  static_assert(XI >= 1 && RB >= 1, "tile shape");
  constexpr int kDmaPerStep = XI + WI;
  constexpr int KUNIT = 1;  // split-K granularity in steps
  constexpr int kDA = TM * DBK * 2, kStage = kDA + DB_BYTES;
  __shared__ __attribute__((aligned(1024))) uint8_t st0[kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t st1[kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t st2[kStage];

  DmaWork wk;
  if (!dma_work(M, N, tail0, tailS, wk, TM)) return;
  const int mblocks = (M + TM - 1) / TM;
  const int nb = wk.lin / mblocks, mb = wk.lin % mblocks;
  const int n0 = nb * DBN, m0 = mb * TM;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int l32 = lane & 31, lh = lane >> 5;
  // split-K over gridDim.y: this workgroup's steps kb .. kb + KS - 1 (whole groups for
  // the group-128 formats); with S > 1 it writes fp32 partials (see the epilogue)
  const int S = wk.S, sp = wk.sp, U = K / (DBK * KUNIT);
  const int kb = KUNIT * (int)((int64_t)sp * U / S), KS = KUNIT * (int)((int64_t)(sp + 1) * U / S) - kb;

  // ---- DMA sources.  x: instruction j covers stage rows 8q .. 8q + 7, q = XI wave + j.
  uint32_t xo[XI];
#pragma unroll
  for (int j = 0; j < XI; ++j) {
    const int r = 8 * (XI * wave + j) + (lane >> 3);
    const int c = (lane & 7) ^ swz_x(r);
    xo[j] = (uint32_t)min(m0 + r, M - 1) * (uint32_t)K + 8 * c;  // M * K < 2^31 (launcher)
  }
  // codes: instruction j covers the 16-row gfx950 tile n0/16 + WI wave + j (rows past
  // N are clamped to the last row).
  const int T = (N + kGemvTileRows - 1) / kGemvTileRows;
  size_t wt_base[WI];
  int wt_nr[WI], wlane[WI];
#pragma unroll
  for (int j = 0; j < WI; ++j) {
    const int t = min(n0 / kGemvTileRows + WI * wave + j, T - 1);
    const int nr = min(kGemvTileRows, N - t * kGemvTileRows);
    wt_base[j] = (size_t)t * kGemvTileRows * K;
    wt_nr[j] = nr;
    wlane[j] = min(lane >> 2, nr - 1);
  }
  const int wc = 16 * ((lane & 3) ^ swz_w(lane >> 2));

  auto code_src = [&](int j, int k0) {
    const int sl = k0 / kSliceBytes, jb = k0 % kSliceBytes;
    const int w = min(kSliceBytes, K - sl * kSliceBytes);
    return qw + wt_base[j] + (size_t)wt_nr[j] * kSliceBytes * sl + wlane[j] * w + jb + wc;
  };
  auto dma = [&](uint8_t* st, int ks) {
    const int k0 = (kb + min(ks, KS - 1)) * DBK;
#pragma unroll
    for (int j = 0; j < XI; ++j) dma16(x + xo[j] + k0, st + (XI * wave + j) * 1024);
#pragma unroll
    for (int j = 0; j < WI; ++j) dma16(code_src(j, k0), st + kDA + (WI * wave + j) * 1024);
  };
  // ---- fragment addresses (bytes within a stage); the swizzles depend only on l32.
  int aaddr[2][2], baddr[2];
#pragma unroll
  for (int P = 0; P < 2; ++P) {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
      aaddr[P][s2] = (wm * 32 * RB + l32) * 128 + 16 * ((4 * P + 2 * lh + s2) ^ swz_x(l32));
    baddr[P] = kDA + (wn * 32 * CB + l32) * 64 + 16 * ((2 * P + lh) ^ swz_w(l32));
  }

  using frag_t = std::conditional_t<XF, h16x8_t, bf16x8_t>;  // eight 16-bit operands
  frag_t A0[2][RB], B0[2][CB];
  frag_t A1[NW == 4 ? 2 : 1][RB], B1[NW == 4 ? 2 : 1][CB];
  auto fread = [&](const uint8_t* st, int P, frag_t (*A)[RB], frag_t (*B)[CB]) {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int i = 0; i < RB; ++i)
        A[s2][i] = *reinterpret_cast<const frag_t*>(st + aaddr[P][s2] + i * 32 * 128);
#pragma unroll
    for (int j = 0; j < CB; ++j) {
      const uint4 raw = *reinterpret_cast<const uint4*>(st + baddr[P] + j * 32 * 64);
      if constexpr (XF) {
        // fp16 (1024 + u) pairs by v_perm_b32 under the exponent byte 0x64, minus 1152 by
        // one packed add: the exact codes q = u - 128, in byte order
        auto q2 = [](uint32_t w, uint32_t sel) {
          return __builtin_bit_cast(uint32_t, __builtin_bit_cast(h16x2_t, __builtin_amdgcn_perm(0x64646464u, w, sel)) +
                                                  h16x2_t{(_Float16)-1152.f, (_Float16)-1152.f});
        };
        B[0][j] = __builtin_bit_cast(frag_t, make_uint4(q2(raw.x, 0x04010400u), q2(raw.x, 0x04030402u),
                                                        q2(raw.y, 0x04010400u), q2(raw.y, 0x04030402u)));
        B[1][j] = __builtin_bit_cast(frag_t, make_uint4(q2(raw.z, 0x04010400u), q2(raw.z, 0x04030402u),
                                                        q2(raw.w, 0x04010400u), q2(raw.w, 0x04030402u)));
      } else {
        B[0][j] = __builtin_bit_cast(frag_t, i8x16_to_bf16_lo(raw));
        B[1][j] = __builtin_bit_cast(frag_t, i8x16_to_bf16_hi(raw));
      }
    }
  };

  floatx16 acc[RB][CB];
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int j = 0; j < CB; ++j)
#pragma unroll
      for (int a = 0; a < 16; ++a) acc[i][j][a] = 0.f;
  auto mma = [&](frag_t (*A)[RB], frag_t (*B)[CB]) {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int j = 0; j < CB; ++j) {
          if constexpr (XF) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[s2][i], B[s2][j], acc[i][j], 0, 0, 0);
          else acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[s2][i], B[s2][j], acc[i][j], 0, 0, 0);
        }
  };
  // This wave's DMA of the step after the current one is complete (only the newest
  // step's kDmaPerStep may still be in flight) and every wave has finished reading
  // the stage that the next DMA overwrites.
  auto step_barrier = [&]() {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(kDmaPerStep) : "memory");
  };

  // Issue order inside a phase: the next slice's LDS reads first, then the MFMAs of
  // the current slice with the code conversions threaded between them, so the matrix
  // core never waits for a burst of VALU work.
  constexpr int kMfmaPerPhase = 2 * RB * CB, kReadsPerPhase = 2 * RB + CB;
  constexpr int kCvtPerPhase = 28 * CB;  // per 16 codes: 4 xor, 16 int -> f32, 8 packs
  constexpr int kLead = kMfmaPerPhase > 4 ? 4 : 1;  // MFMAs that cover the LDS read latency
  constexpr int kv = (kCvtPerPhase + kMfmaPerPhase - kLead - 1) / (kMfmaPerPhase - kLead) + 1;
  auto phase_order = [&]() {
    __builtin_amdgcn_sched_group_barrier(0x100, kReadsPerPhase, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, kLead, 0);
#pragma unroll
    for (int i = kLead; i < kMfmaPerPhase; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, kv, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  dma(st0, 0);
  dma(st1, 1);
  dma(st2, 2);
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(2 * kDmaPerStep) : "memory");
  // Four waves (one per SIMD) software-pipeline their fragment reads one slice ahead
  // (two fragment sets); with eight waves (two per SIMD) the registers hold one set and
  // the other wave on the SIMD covers the LDS latency.
  constexpr bool kPipelined = NW == 4;
  if constexpr (kPipelined) fread(st0, 0, A0, B0);
  auto step = [&](uint8_t* cur, uint8_t* nxt, int t) {
    if constexpr (kPipelined) {
      fread(cur, 1, A1, B1);
      mma(A0, B0);
      phase_order();
      step_barrier();
      dma(cur, t + 3);  // every wave is done with this stage
      __builtin_amdgcn_sched_barrier(0);
      fread(nxt, 0, A0, B0);
      mma(A1, B1);
      phase_order();
    } else {
      (void)nxt;
      fread(cur, 0, A0, B0);
      mma(A0, B0);
      fread(cur, 1, A0, B0);
      mma(A0, B0);
      step_barrier();
      dma(cur, t + 3);
    }
  };
  // Three steps per iteration keep every stage address static; the K % 3 steps left
  // over run after the loop (an early exit inside the loop body makes the register
  // allocator spill the accumulators).
  const int KS3 = KS - KS % 3;
  for (int t = 0; t < KS3; t += 3) {
    step(st0, st1, t);
    step(st1, st2, t + 1);
    step(st2, st0, t + 2);
  }
  if (KS % 3 >= 1) step(st0, st1, KS3);
  if (KS % 3 == 2) step(st1, st2, KS3 + 1);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---- epilogue: D[row = 8*(a/4) + 4*(lane/32) + a%4][col = lane%32] of each 32x32 block;
  // split-K ranges write raw fp32 partials (the reduction applies the scale)
#pragma unroll
  for (int j = 0; j < CB; ++j) {
    const int n = n0 + wn * 32 * CB + j * 32 + l32;
    if (n >= N) continue;
    const float sc = bf16_to_f32(scales[n]);
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
      for (int a = 0; a < 16; ++a) {
        const int m = m0 + wm * 32 * RB + i * 32 + 8 * (a >> 2) + 4 * lh + (a & 3);
        if (m >= M) continue;
        if (S == 1) y[(size_t)m * N + n] = f32_to_out<XF>(with_res<XF>(sc * acc[i][j][a], res, (size_t)m * N + n));
        else part[wk.poff + (size_t)(m - wk.pm0) * wk.ppitch + (n - wk.pn0)] = acc[i][j][a];
      }
  }
}

template <int WM, int WN, bool XF = false>
__global__ __launch_bounds__(64 * WM * WN, 1) void gemm_dma_w8pc_kernel(const uint8_t* __restrict__ qw,
                                                                         const uint16_t* __restrict__ scales,
                                                                         const uint16_t* __restrict__ x,
                                                                         uint16_t* y,
                                                                         float* __restrict__ part, int M, int K,
                                                                         int N, int tail0, int tailS,
                                                                         const uint16_t* res) {
  dma_w8pc_body<WM, WN, DBM, XF>(qw, scales, x, y, part, M, K, N, tail0, tailS, res);
}

// 64- and 128-row tiles (capping the registers for two workgroups per CU spills:
// measured slower)
template <int TM, bool XF = false>
__global__ __launch_bounds__(512, 1) void gemm_dma64_w8pc_kernel(const uint8_t* __restrict__ qw, const uint16_t* __restrict__ scales,
                            const uint16_t* __restrict__ x, uint16_t* y, float* __restrict__ part,
                            int M, int K, int N, int tail0, int tailS, const uint16_t* res) {
  dma_w8pc_body<1, 8, TM, XF>(qw, scales, x, y, part, M, K, N, tail0, tailS, res);
}

// ---------------------------------------------------------------------------------
// Group-128 formats: the same LDS-DMA pipeline with fp16 matrix products of exact
// factors.
//
// A group scale cannot stay outside the products the way a per-channel scale does, and
// neither bf16 nor fp16 holds s (q - z) exactly (rounding every weight to bf16 costs up
// to 0.9 of the tolerance at K = 5120, growing with sqrt(K); fp16 rounds 8x finer but
// its worst case still exceeds the tolerance wherever products cancel).  So the B
// fragments are the exact codes -- under an fp16 exponent pattern (v_perm_b32 for int8:
// 1024 + u; v_and_or_b32 for uint4: 1024 + q from bits 0..3 of a half, 64 + q from bits
// 4..7), the offset and zero-point removed exactly by one packed fp16 add -- against x
// in fp16, and a second accumulator set takes each group's partial sums, which are added
// into the first times the group's scale (fp32) when the group ends.  Every product is
// exact, so an output carries only fp32 summation and the final bf16 rounding.  The
// second set is why these tiles are 128 x 256 (eight waves of 128 x 32, or 64 x 32 for
// the 64-row tiles): at 256 x 256 the two sets exceed the registers of two waves per SIMD.
//
// x reaches the matrix cores in fp16: converted once per call by x_to_f16_rows_kernel
// when the workspace has room -- each row scaled by a power of two so that all of it
// converts exactly, the scale taken back out in the epilogue -- otherwise in LDS,
// unscaled, once per step and workgroup (every lane converts the 16-byte chunks its own
// DMA brought, right after waiting for them, so the step's one barrier also covers the
// conversion).  A value fp16 cannot hold exactly (unscaled: other than 0 or 2^-17 <= |x|
// <= 65280) converts to NaN, so that the tile's accumulators end non-finite and the
// workgroup recomputes its tile on the exact path (bf16 codes q or q - z against bf16 x,
// fp32 partial per group times the scale, operands straight from memory: slow, and only
// for such inputs).
//
// A stage also holds the step's group metadata (the 256 rows' scales and, for uint4,
// zero-points), brought by one more LDS-DMA of waves 0 and 1.  uint4 codes take 32
// bytes per row and step; chunk c of row n sits at position c ^ ((n >> 3) & 1).
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

// The LDS-DMA with 4-byte lanes (lane i writes LDS byte l + 4 i).
__device__ __forceinline__ void dma4(const void* g, uint8_t* l) {
  const uint32_t la = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)l);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off" ::"s"(la), "v"(g) : "memory", "m0");
}

// GS: k per group (128, or 64 / 32 for the smaller groups: a step of DBK = 64 k then
// holds kGPS = 1 or 2 whole groups, and its stage their metadata side by side)
template <int FMT, int TM = DBM, int GS = kGroup>
struct G128Dma {
  static constexpr bool kW4 = FMT == WQ_FMT_W4_G128;
  static constexpr int kGPS = GS >= DBK ? 1 : DBK / GS;  // groups whose metadata a stage holds
  static constexpr int kXBytes = TM * DBK * 2;          // x rows of a stage
  static constexpr int kCodeRow = kW4 ? DBK / 2 : DBK;  // code bytes per row and step
  static constexpr int kCodeBytes = DBN * kCodeRow;
  static constexpr int kMetaBytes = kGPS * (DBN * 2 + (kW4 ? DBN / 2 : 0));
  static constexpr int kStage = kXBytes + kCodeBytes + kMetaBytes;
  static constexpr int kCodeInst = kCodeBytes / 1024;  // code DMA instructions per step
};

// Exact fallback for one workgroup tile (see above): each wave takes 32 x 32 blocks in
// turn; per block and group, eight v_mfma_f32_32x32x16_bf16 on exact codes give the
// group's fp32 partial, which the group scale adds into the block.
// (g0, g1: the K range in units of 128 k; the groups of GS k inside it, in order)
template <int FMT, int TM = DBM, int GS = kGroup>
__device__ void g128_tile_exact(const uint8_t* __restrict__ qw, const uint16_t* __restrict__ scales,
                                const uint8_t* __restrict__ zeros, const uint16_t* __restrict__ x,
                                uint16_t* y, float* __restrict__ part, int M, int K, int N,
                                int m0, int n0, int g0, int g1, int S, size_t poff, int ppitch, int pm0,
                                int pn0, int wave, int NW, const uint16_t* res) {
  constexpr bool kW4 = FMT == WQ_FMT_W4_G128;
  const int lane = threadIdx.x & 63, l32 = lane & 31, lh = lane >> 5;
  const int G = K / GS;
  const int row_bytes = kW4 ? K / 2 : K;
  for (int blk = wave; blk < (TM / 32) * (DBN / 32); blk += NW) {
    const int bi = blk / (DBN / 32), bj = blk % (DBN / 32);
    const int m = min(m0 + 32 * bi + l32, M - 1), n = min(n0 + 32 * bj + l32, N - 1);
    const size_t mi = ((size_t)(n / kGemvTileRows) * G) * kGemvTileRows + n % kGemvTileRows;
    floatx16 acc;
#pragma unroll
    for (int a = 0; a < 16; ++a) acc[a] = 0.f;
    for (int g = g0 * (kGroup / GS); g < g1 * (kGroup / GS); ++g) {
      const uint16_t sb = scales[mi + (size_t)g * kGemvTileRows];
      const float sc = kW4 ? f16_to_f32(sb) : bf16_to_f32(sb);
      float z = 0.f;
      if constexpr (kW4) z = (float)((zeros[(mi + (size_t)g * kGemvTileRows) / 2] >> (4 * (n & 1))) & 15u);
      floatx16 tmp;
#pragma unroll
      for (int a = 0; a < 16; ++a) tmp[a] = 0.f;
      for (int kk = 0; kk < GS / 16; ++kk) {
        const int k = g * GS + 16 * kk + 8 * lh;
        const uint4 xa = *reinterpret_cast<const uint4*>(x + (size_t)m * K + k);
        uint4 wb;
        if constexpr (kW4) {
          wb = w4_word_to_bf16(*reinterpret_cast<const uint32_t*>(qw + tiled_offset(n, k / 2, N, row_bytes)), z);
        } else {
          const uint2 c = *reinterpret_cast<const uint2*>(qw + tiled_offset(n, k, N, row_bytes));
          wb = i8x16_to_bf16_lo(make_uint4(c.x, c.y, 0u, 0u));
        }
        tmp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, xa),
                                                      __builtin_bit_cast(bf16x8_t, wb), tmp, 0, 0, 0);
      }
#pragma unroll
      for (int a = 0; a < 16; ++a) acc[a] = fmaf(sc, tmp[a], acc[a]);
    }
    const int nn = n0 + 32 * bj + l32;
    if (nn >= N) continue;
#pragma unroll
    for (int a = 0; a < 16; ++a) {
      const int mm = m0 + 32 * bi + 8 * (a >> 2) + 4 * lh + (a & 3);
      if (mm >= M) continue;
      if (S == 1) y[(size_t)mm * N + nn] = f32_to_out<false>(with_res<false>(acc[a], res, (size_t)mm * N + nn));
      else part[poff + (size_t)(mm - pm0) * ppitch + (nn - pn0)] = acc[a];
    }
  }
}

// Eight bf16 values -> fp16, each exactly, or NaN where fp16 cannot hold the value
// exactly (0 < |x| < 2^-17, |x| > 65280, Inf, NaN): a NaN makes the tile's accumulators
// non-finite, which sends the tile down the exact path, so the fp16 operands are
// always the activations themselves.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2_exact(uint32_t w) {
  const float2_t f = {__uint_as_float(w << 16), __uint_as_float(w & 0xFFFF0000u)};
  uint32_t o = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2_t));
  const uint32_t lo = w & 0x7FFFu, hi = (w >> 16) & 0x7FFFu;
  if (lo != 0 && (lo < 0x3700u || lo > 0x477Fu)) o = (o & 0xFFFF0000u) | 0x7E00u;
  if (hi != 0 && (hi < 0x3700u || hi > 0x477Fu)) o = (o & 0x0000FFFFu) | 0x7E000000u;
  return o;
}
__device__ __forceinline__ uint4 bf16x8_to_f16x8(uint4 v) {
  return make_uint4(bf16x2_to_f16x2_exact(v.x), bf16x2_to_f16x2_exact(v.y), bf16x2_to_f16x2_exact(v.z),
                    bf16x2_to_f16x2_exact(v.w));
}

// x converted to fp16 once per call for the group-128 LDS-DMA tiles when the workspace
// has room, one workgroup per row, each row scaled by a power of two 2^e_m chosen from
// its largest and smallest nonzero magnitude so that every value converts exactly: the
// largest lands below 2^15, and the row is exact when its smallest nonzero value then
// lands at 2^-17 or above (a spread of up to 2^31 between them; activations drawn from
// N(0, 1) hold values near 1e-6, which unscaled fp16 cannot hold).  xinv[m] = 2^-e_m
// takes the scale back out of the fp32 results, exactly.  A row that cannot be held
// (a wider spread, a bf16 subnormal, Inf or NaN) is written as NaN, so that its tiles
// recompute on the exact path.  Otherwise every workgroup converts the x chunks of each
// stage it loads (no scaling: tiles whose x fp16 cannot hold fall back).
// One workgroup per row, up to 1024 threads: each thread keeps its first kXRowRegs 16-byte
// chunks in registers between the two passes (rows up to 32768 k are read once, every
// load issued before the first is used); longer rows read the rest again.
constexpr int kXRowRegs = 4;
__global__ __launch_bounds__(1024) void x_to_f16_rows_kernel(const uint16_t* __restrict__ x, uint16_t* __restrict__ xh,
                                                             float* __restrict__ xinv, int K) {
  __shared__ uint32_t red_mx[16], red_mn[16];
  const int m = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T = blockDim.x, NWv = T >> 6;
  const uint4* xr = reinterpret_cast<const uint4*>(x + (size_t)m * K);
  uint4* xo = reinterpret_cast<uint4*>(xh + (size_t)m * K);
  const int n8 = K / 8;
  uint32_t mx = 0, mn = 0xFFFFu;  // largest |x| bits, smallest nonzero |x| bits
  auto scan = [&](const uint4& v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t lo = w[q] & 0x7FFFu, hi = (w[q] >> 16) & 0x7FFFu;
      mx = max(mx, max(lo, hi));
      mn = min(mn, min(lo ? lo : 0xFFFFu, hi ? hi : 0xFFFFu));
    }
  };
  uint4 keep[kXRowRegs];
#pragma unroll
  for (int j = 0; j < kXRowRegs; ++j) {
    const int i = tid + j * T;
    keep[j] = i < n8 ? xr[i] : make_uint4(0u, 0u, 0u, 0u);  // zeros change neither bound
  }
#pragma unroll
  for (int j = 0; j < kXRowRegs; ++j) scan(keep[j]);
  for (int i = tid + kXRowRegs * T; i < n8; i += T) scan(xr[i]);
  for (int d = 32; d >= 1; d >>= 1) {
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, d));
    mn = min(mn, (uint32_t)__shfl_xor((int)mn, d));
  }
  if (lane == 0) {
    red_mx[wave] = mx;
    red_mn[wave] = mn;
  }
  __syncthreads();
  mx = red_mx[0];
  mn = red_mn[0];
  for (int w = 1; w < NWv; ++w) {
    mx = max(mx, red_mx[w]);
    mn = min(mn, red_mn[w]);
  }
  // biased bf16 exponents; the scale puts the largest value below 2^15 (e capped so
  // that 2^-e stays a normal fp32 number)
  const int emax = (int)(mx >> 7), emin = (int)(mn >> 7);
  const int e = mx == 0 ? 0 : min(141 - emax, 100);
  const bool ok = mx == 0 || (emax < 255 && emax + e <= 141 && (mn == 0xFFFFu || (emin >= 1 && emin + e >= 110)));
  const float sc = __builtin_bit_cast(float, (uint32_t)(127 + e) << 23);  // 2^e, -113 <= e <= 100
  auto conv = [&](const uint4& v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float2_t f = {__uint_as_float(w[q] << 16) * sc, __uint_as_float(w[q] & 0xFFFF0000u) * sc};
      o[q] = ok ? __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2_t)) : 0x7E007E00u;
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
  };
#pragma unroll
  for (int j = 0; j < kXRowRegs; ++j) {
    const int i = tid + j * T;
    if (i < n8) xo[i] = conv(keep[j]);
  }
  for (int i = tid + kXRowRegs * T; i < n8; i += T) xo[i] = conv(xr[i]);
  if (tid == 0) xinv[m] = __builtin_bit_cast(float, (uint32_t)(127 - e) << 23);  // 2^-e
}

// XH: xd is x already in fp16, row m scaled by 1 / xinv[m] (x_to_f16_rows_kernel);
// otherwise xd == x and the stages are converted in LDS.  The exact fallback always
// reads the bf16 x.
// XF: fp16 activations -- x arrives as fp16 (passed as xd, with XH), needs no row
// scale, no exact fallback (fp16 x times exact fp16 codes is exact in fp32), and y is fp16.
template <int FMT, int WM, int WN, bool XH = false, int TM = DBM, int GS = kGroup, bool XF = false>
__global__ __launch_bounds__(64 * WM * WN, 1) void gemm_dma_g128_kernel(const uint8_t* __restrict__ qw,
                                                                         const uint16_t* __restrict__ scales,
                                                                         const uint8_t* __restrict__ zeros,
                                                                         const uint16_t* __restrict__ x,
                                                                         const uint16_t* __restrict__ xd,
                                                                         const float* __restrict__ xinv,
                                                                         uint16_t* y,
                                                                         float* __restrict__ part, int M, int K,
                                                                         int N, int tail0,
                                                                         int tailS, const uint16_t* res) {
  using F = G128Dma<FMT, TM, GS>;
  constexpr bool kW4 = F::kW4;
  constexpr int NW = WM * WN, RB = TM / 32 / WM, CB = 8 / WN;
  constexpr int XI = TM / 8 / NW, WI = F::kCodeInst / NW;  // x and code DMA instructions per wave and step
  constexpr int kDA = F::kXBytes;
  static_assert(XI >= 1 && RB >= 1, "tile shape");
  constexpr int kDmaPerStep = XI + WI;
  constexpr int KUNIT = 2;  // split-K granularity in steps: one group
  static_assert(WI >= 1, "every wave takes part in the code DMA");
  static_assert(NW == 8, "eight waves: each holds one 16-k half of a slice at a time");
  __shared__ __attribute__((aligned(1024))) uint8_t st0[F::kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t st1[F::kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t st2[F::kStage];
  __shared__ int wave_flag[NW];

  DmaWork wk;
  if (!dma_work(M, N, tail0, tailS, wk, TM)) return;
  const int mblocks = (M + TM - 1) / TM;
  const int nb = wk.lin / mblocks, mb = wk.lin % mblocks;
  const int n0 = nb * DBN, m0 = mb * TM;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int l32 = lane & 31, lh = lane >> 5;
  // split-K over gridDim.y: this workgroup's steps kb .. kb + KS - 1 (whole groups for
  // the group-128 formats); with S > 1 it writes fp32 partials (see the epilogue)
  const int S = wk.S, sp = wk.sp, U = K / (DBK * KUNIT);
  const int kb = KUNIT * (int)((int64_t)sp * U / S), KS = KUNIT * (int)((int64_t)(sp + 1) * U / S) - kb;
  const int G = K / GS;
  const int row_bytes = kW4 ? K / 2 : K;

  // ---- DMA sources.  x: instruction j covers stage rows 8q .. 8q + 7, q = XI wave + j.
  uint32_t xo[XI];
#pragma unroll
  for (int j = 0; j < XI; ++j) {
    const int r = 8 * (XI * wave + j) + (lane >> 3);
    const int c = (lane & 7) ^ swz_x(r);
    xo[j] = (uint32_t)min(m0 + r, M - 1) * (uint32_t)K + 8 * c;  // M * K < 2^31 (launcher)
  }
  // codes: int8 instruction j covers the 16-row tile n0/16 + WI wave + j (16 rows x 64
  // bytes), uint4 instruction j the two tiles from n0/16 + 2 (WI wave + j) (32 rows x 32
  // bytes, lanes 0..31 the first).  Rows past N are clamped to the last row.
  constexpr int kTilesPerInst = kW4 ? 2 : 1;
  const int T = (N + kGemvTileRows - 1) / kGemvTileRows;
  size_t wt_base[WI];
  int wt_nr[WI], wlane[WI];
#pragma unroll
  for (int j = 0; j < WI; ++j) {
    const int t = min(n0 / kGemvTileRows + kTilesPerInst * (WI * wave + j) + (kW4 ? lane >> 5 : 0), T - 1);
    const int nr = min(kGemvTileRows, N - t * kGemvTileRows);
    wt_base[j] = (size_t)t * kGemvTileRows * row_bytes;
    wt_nr[j] = nr;
    wlane[j] = min(kW4 ? (lane >> 1) & 15 : lane >> 2, nr - 1);
  }
  const int wc = kW4 ? 16 * ((lane & 1) ^ ((lane >> 4) & 1)) : 16 * ((lane & 3) ^ swz_w(lane >> 2));
  auto code_src = [&](int j, int k0) {
    const int b0 = kW4 ? k0 / 2 : k0;  // byte of the packed row
    const int sl = b0 / kSliceBytes, jb = b0 % kSliceBytes;
    const int w = min(kSliceBytes, row_bytes - sl * kSliceBytes);
    return qw + wt_base[j] + (size_t)wt_nr[j] * kSliceBytes * sl + wlane[j] * w + jb + wc;
  };
  // metadata: wave 0 brings the 16 tiles' scales of the step's group (2 lanes x 16
  // bytes per tile; lanes 32.. the second group of a step of two), wave 1 the uint4
  // zero-points (2 lanes x 4 bytes per tile)
  const int mt = min(n0 / kGemvTileRows + ((lane & 31) >> 1), T - 1);
  auto dma = [&](uint8_t* st, int ks) {
    const int k0 = (kb + min(ks, KS - 1)) * DBK;
#pragma unroll
    for (int j = 0; j < XI; ++j) dma16(xd + xo[j] + k0, st + (XI * wave + j) * 1024);
#pragma unroll
    for (int j = 0; j < WI; ++j) dma16(code_src(j, k0), st + kDA + (WI * wave + j) * 1024);
    const int g = k0 / GS + (F::kGPS > 1 ? lane >> 5 : 0);
    if (wave == 0 && lane < 32 * F::kGPS)
      dma16(scales + ((size_t)mt * G + g) * kGemvTileRows + 8 * (lane & 1), st + kDA + F::kCodeBytes);
    if (kW4 && wave == 1 && lane < 32 * F::kGPS)
      dma4(zeros + ((size_t)mt * G + g) * (kGemvTileRows / 2) + 4 * (lane & 1),
           st + kDA + F::kCodeBytes + F::kGPS * DBN * 2);
  };
  // the x chunks this lane's own DMA brought into a stage, bf16 -> fp16 in place
  // (v_cvt_pk_f16_f32, nearest even: beyond fp16 range gives Inf)
  // (nothing to do when x arrives as fp16: XH, converted by x_to_f16_rows_kernel)
  auto convert = [&](uint8_t* st) {
    if constexpr (XH) return;
#pragma unroll
    for (int j = 0; j < XI; ++j) {
      uint4* p = reinterpret_cast<uint4*>(st + (XI * wave + j) * 1024 + 16 * lane);
      *p = bf16x8_to_f16x8(*p);
    }
  };
  // ---- fragment addresses (bytes within a stage); the swizzles depend only on l32.
  int aaddr[2][2], baddr[2];
#pragma unroll
  for (int P = 0; P < 2; ++P) {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
      aaddr[P][s2] = (wm * 32 * RB + l32) * 128 + 16 * ((4 * P + 2 * lh + s2) ^ swz_x(l32));
    if constexpr (kW4)
      baddr[P] = kDA + (wn * 32 * CB + l32) * 32 + 16 * (P ^ ((l32 >> 3) & 1)) + 8 * lh;
    else
      baddr[P] = kDA + (wn * 32 * CB + l32) * 64 + 16 * ((2 * P + lh) ^ swz_w(l32));
  }

  // the step's group metadata for this lane's CB columns: the scale in fp32 (exact),
  // and minus the code offset plus zero-point as fp16 pairs (uint4: 1024 + z and 64 + z;
  // int8: 1152)
  float msc[CB];
  f16x2_t mo0[CB], mo1[CB];
  auto meta_read = [&](const uint8_t* st, int gi) {
#pragma unroll
    for (int j = 0; j < CB; ++j) {
      const int n = wn * 32 * CB + j * 32 + l32;
      const uint16_t sb = *reinterpret_cast<const uint16_t*>(st + kDA + F::kCodeBytes + gi * DBN * 2 + 2 * n);
      if constexpr (kW4) {
        const uint8_t zb = st[kDA + F::kCodeBytes + F::kGPS * DBN * 2 + gi * (DBN / 2) + (n >> 1)];
        const _Float16 z = (_Float16)(float)((zb >> (4 * (n & 1))) & 15u);
        msc[j] = f16_to_f32(sb);
        mo0[j] = f16x2_t{-(_Float16)1024.f - z, -(_Float16)1024.f - z};
        mo1[j] = f16x2_t{-(_Float16)64.f - z, -(_Float16)64.f - z};
      } else {
        msc[j] = bf16_to_f32(sb);
        mo0[j] = f16x2_t{(_Float16)-1152.f, (_Float16)-1152.f};
      }
    }
  };
  uint32_t nib_lo = 0x000F000Fu, nib_hi = 0x00F000F0u, mag_1024 = 0x64006400u, mag_64 = 0x54005400u;
  if constexpr (kW4) asm volatile("" : "+v"(nib_lo), "+v"(nib_hi), "+s"(mag_1024), "+s"(mag_64));
  // fp16 pair (offset + q) -> fp16 pair (q - z), or q for int8: one exact add
  auto deq = [&](uint32_t h, f16x2_t off) -> uint32_t {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, h) + off);
  };
  // One half s2 of a slice (eight waves: the registers hold one half at a time): the A
  // fragments of MFMA s2 and the B fragments they meet.
  auto fread_half = [&](const uint8_t* st, int P, int s2, f16x8_t* A, f16x8_t* B) {
#pragma unroll
    for (int i = 0; i < RB; ++i) A[i] = *reinterpret_cast<const f16x8_t*>(st + aaddr[P][s2] + i * 32 * 128);
    // the group's metadata where a group starts: each step for 128 and 64 (a group-128
    // step re-reads its group's), each 32-k slice P for 32
    if (s2 == 0 && (P == 0 || F::kGPS > 1)) meta_read(st, F::kGPS > 1 ? P : 0);
#pragma unroll
    for (int j = 0; j < CB; ++j) {
      if constexpr (kW4) {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(st + baddr[P] + j * 32 * 32 + 4 * s2), w8 = w >> 8;
        const uint4 o = make_uint4(deq((w & nib_lo) | mag_1024, mo0[j]),
                                   deq((w & nib_hi) | mag_64, mo1[j]),
                                   deq((w8 & nib_lo) | mag_1024, mo0[j]),
                                   deq((w8 & nib_hi) | mag_64, mo1[j]));
        B[j] = __builtin_bit_cast(f16x8_t, o);
      } else {
        const uint2 raw = *reinterpret_cast<const uint2*>(st + baddr[P] + j * 32 * 64 + 8 * s2);
        const uint4 o = make_uint4(deq(__builtin_amdgcn_perm(0x64646464u, raw.x, 0x04010400u), mo0[j]),
                                   deq(__builtin_amdgcn_perm(0x64646464u, raw.x, 0x04030402u), mo0[j]),
                                   deq(__builtin_amdgcn_perm(0x64646464u, raw.y, 0x04010400u), mo0[j]),
                                   deq(__builtin_amdgcn_perm(0x64646464u, raw.y, 0x04030402u), mo0[j]));
        B[j] = __builtin_bit_cast(f16x8_t, o);
      }
    }
  };

  // acc: the scaled sum over the groups so far; grp: the current group's partial sums
  // of exact products, added into acc times the group scale when the group ends
  floatx16 acc[RB][CB], grp[RB][CB];
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int j = 0; j < CB; ++j)
#pragma unroll
      for (int a = 0; a < 16; ++a) {
        acc[i][j][a] = 0.f;
        grp[i][j][a] = 0.f;
      }
  auto mma_half = [&](const f16x8_t* A, const f16x8_t* B) {
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
      for (int j = 0; j < CB; ++j)
        grp[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[i], B[j], grp[i][j], 0, 0, 0);
  };
  auto fold = [&]() {
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
      for (int j = 0; j < CB; ++j)
#pragma unroll
        for (int a = 0; a < 16; ++a) {
          acc[i][j][a] = fmaf(msc[j], grp[i][j][a], acc[i][j][a]);
          grp[i][j][a] = 0.f;
        }
  };
  // This wave's DMA of the step after the current one is complete (only the newest
  // step's kDmaPerStep may still be in flight; waves 0 and 1 issue one more, so they
  // wait for one instruction more than needed); its x chunks are converted; then
  // every wave has converted its chunks and finished reading the stage that the next
  // DMA overwrites.
  auto step_barrier = [&](uint8_t* nxt) {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kDmaPerStep) : "memory");
    convert(nxt);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };

  dma(st0, 0);
  dma(st1, 1);
  dma(st2, 2);
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * kDmaPerStep) : "memory");
  convert(st0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  // one step: both 32-k slices, a half (16 k) at a time (the registers hold one half);
  // a group of 128 is two steps (the range starts on a group), so odd steps end one; a
  // group of 64 ends with every step, one of 32 with every slice
  auto step = [&](uint8_t* cur, uint8_t* nxt, int t) {
    f16x8_t Ah[RB], Bh[CB];
#pragma unroll
    for (int P = 0; P < 2; ++P) {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        fread_half(cur, P, s2, Ah, Bh);
        mma_half(Ah, Bh);
      }
      if constexpr (GS == 32) {
        if (KS > 0) fold();  // (always true: the branch keeps the fold in a block of its own)
      }
    }
    if constexpr (GS == 64) {
      if (KS > 0) fold();
    }
    if constexpr (GS == kGroup) {
      if (t & 1) fold();
    }
    step_barrier(nxt);
    dma(cur, t + 3);
  };
  const int KS3 = KS - KS % 3;
  for (int t = 0; t < KS3; t += 3) {
    step(st0, st1, t);
    step(st1, st2, t + 1);
    step(st2, st0, t + 2);
  }
  if (KS % 3 >= 1) step(st0, st1, KS3);
  if (KS % 3 == 2) step(st1, st2, KS3 + 1);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---- a non-finite accumulator (an x that fp16 cannot hold exactly arrives as NaN,
  // and beyond fp16's range products overflow) sends the tile down the exact path
  // (fp16 activations are the operands themselves: their results stand as computed)
  if constexpr (!XF) {
    bool bad = false;
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
      for (int j = 0; j < CB; ++j)
#pragma unroll
        for (int a = 0; a < 16; ++a) bad |= !__builtin_isfinite(acc[i][j][a]);
    const bool wave_bad = __builtin_amdgcn_ballot_w64(bad) != 0;
    if (lane == 0) wave_flag[wave] = wave_bad ? 1 : 0;
    __syncthreads();
    int any = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) any |= wave_flag[w];
    if (any) {
      g128_tile_exact<FMT, TM, GS>(qw, scales, zeros, x, y, part, M, K, N, m0, n0, kb / KUNIT, (kb + KS) / KUNIT,
                                   S, wk.poff, wk.ppitch, wk.pm0, wk.pn0, wave, NW, res);
      return;
    }
  }
  // ---- epilogue: D[row = 8*(a/4) + 4*(lane/32) + a%4][col = lane%32] of each 32x32 block;
  // split-K ranges write fp32 partials
#pragma unroll
  for (int j = 0; j < CB; ++j) {
    const int n = n0 + wn * 32 * CB + j * 32 + l32;
    if (n >= N) continue;
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
      for (int a = 0; a < 16; ++a) {
        const int m = m0 + wm * 32 * RB + i * 32 + 8 * (a >> 2) + 4 * lh + (a & 3);
        if (m >= M) continue;
        const float v = XH && !XF ? acc[i][j][a] * xinv[m] : acc[i][j][a];  // the row's scale back out (exact)
        if (S == 1) y[(size_t)m * N + n] = f32_to_out<XF>(with_res<XF>(v, res, (size_t)m * N + n));
        else part[wk.poff + (size_t)(m - wk.pm0) * wk.ppitch + (n - wk.pn0)] = v;
      }
  }
}

// ---------------------------------------------------------------------------------
// Skinny GEMM, 8 <= M <= 128 tokens.  At these M the layer is still bound by the
// weight stream (2 M flops per int8 byte), so the kernel is built like the decode
// GEMV with the dot products moved onto the matrix cores:
//
//   * a workgroup owns 128 weight rows (4 waves x 2 tiles of 16) and a range of K
//     (split-K over gridDim.y: fp32 partials, summed in order by a second kernel);
//   * each wave loads its codes straight from memory into registers -- no weight
//     byte is used by two waves, so LDS would only add a round trip.  One 16-byte
//     load per lane covers 16 rows x 64 k (W8) or 16 rows x 128 k (W4) of a tile;
//   * the x slice of a K step (TB*16 tokens x 128 k, bf16) goes through LDS once per
//     workgroup and feeds all four waves (17 <= M; one token block takes the direct
//     kernel below);
//   * v_mfma_f32_16x16x32_bf16 with x as the A operand (16 tokens) and the exact
//     bf16 codes as B (16 weight rows).  Lane group c (lanes 16c .. 16c+15) of MFMA s
//     takes k = 16c + 8s + 0..7 (W8, per 64 k) or 32c + 8s + 0..7 (W4, per 128 k), so
//     a lane's 16-byte code chunk feeds 2 (W8) or 4 (W4) MFMAs; x is read with the
//     same permutation;
//   * a K step is 128 = one group: group-128 formats add s[n][g] times the step's fp32
//     partial to the accumulator; per-channel W8 scales at the end.
constexpr int SK_ROWS = 128, SK_STEP = 128;
constexpr int SK_XP = SK_STEP * 2 + 16;  // LDS pitch of one token's x slice, bytes (16-byte pad)

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int FMT, int TB>
__global__ __launch_bounds__(256) void gemm_skinny_kernel(const uint8_t* __restrict__ qw,
                                                           const uint16_t* __restrict__ scales,
                                                           const uint8_t* __restrict__ zeros,
                                                           const uint16_t* __restrict__ x,
                                                           uint16_t* y, float* __restrict__ part,
                                                           int M, int K, int N, int S, const uint16_t* res) {
  constexpr bool kW4 = FMT == WQ_FMT_W4_G128, kGrouped = FMT != WQ_FMT_W8_PC;
  constexpr int RT = 2;                  // 16-row tiles per wave
  constexpr int CH = kW4 ? 1 : 2;        // 16-byte code chunks per lane, tile and step
  constexpr int XJ = TB;                 // x chunks (16 bytes) per thread and step
  __shared__ __attribute__((aligned(16))) uint8_t xs[2][TB * 16 * SK_XP];
  constexpr int kTrPitch = SK_STEP + 16;  // LDS pitch of a transposed code row (bytes, padded)
  __shared__ __attribute__((aligned(16))) uint8_t trs[4][kW4 ? 1 : RT * 16 * kTrPitch];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, c4 = lane >> 4;
  const int n0 = blockIdx.x * SK_ROWS;
  const int KS = K / SK_STEP, G = K / kGroup;
  const int ks0 = (int)((int64_t)KS * blockIdx.y / S), ks1 = (int)((int64_t)KS * (blockIdx.y + 1) / S);
  const int64_t row_bytes = kW4 ? K / 2 : K;

  int nrow[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) nrow[t] = min(n0 + wave * 32 + t * 16 + r16, N - 1);

  // x staging: chunk c = tid + 256 j is token c / 16, bf16 elements 8 (c % 16) .. + 7.
  auto xload = [&](u32x4* xr, int ks) {
#pragma unroll
    for (int j = 0; j < XJ; ++j) {
      const int c = tid + 256 * j;
      const int m = min(c >> 4, M - 1);  // tokens past M feed only outputs never stored
      xr[j] = *reinterpret_cast<const u32x4*>(x + (size_t)m * K + ks * SK_STEP + (c & 15) * 8);
    }
  };
  auto xstore = [&](const u32x4* xr, int buf) {
#pragma unroll
    for (int j = 0; j < XJ; ++j) {
      const int c = tid + 256 * j;
      *reinterpret_cast<u32x4*>(&xs[buf][(c >> 4) * SK_XP + (c & 15) * 16]) = xr[j];
    }
  };
  uint4 cw[RT][CH];
  // W4: lane l loads row l % 16, chunk l / 16 (the fragment layout).  W8: lane l loads
  // row l / 8 + 8 j, chunk l % 8 -- whole 128-byte lines per instruction -- and the
  // chunks reach the fragment layout through the wave's own LDS area (transpose()).
  auto code_ptr = [&](int t, int j, int ks) {
    if constexpr (kW4) {
      return reinterpret_cast<const uint4*>(qw + tiled_offset(nrow[t], (int64_t)ks * (SK_STEP / 2) + 16 * c4, N, row_bytes));
    } else {
      const int rr = min(n0 + wave * 32 + t * 16 + (lane >> 3) + 8 * j, N - 1);
      return reinterpret_cast<const uint4*>(qw + tiled_offset(rr, (int64_t)ks * SK_STEP + 16 * (lane & 7), N, row_bytes));
    }
  };
  auto transpose = [&](uint4 (*c)[CH]) {
    if constexpr (!kW4) {
      uint8_t* tw = trs[wave];
#pragma unroll
      for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int i = 0; i < CH; ++i)
          *reinterpret_cast<uint4*>(tw + (t * 16 + (lane >> 3) + 8 * i) * kTrPitch + 16 * (lane & 7)) = c[t][i];
#pragma unroll
      for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int j = 0; j < CH; ++j)
          c[t][j] = *reinterpret_cast<const uint4*>(tw + (t * 16 + r16) * kTrPitch + 16 * (4 * j + c4));
    }
  };
  auto gscale = [&](int n, int g) -> float {
    const uint16_t sb = scales[((size_t)(n / kGemvTileRows) * G + g) * kGemvTileRows + n % kGemvTileRows];
    return (FMT == WQ_FMT_W8_G128) ? bf16_to_f32(sb) : f16_to_f32(sb);
  };

  floatx4 acc[RT][TB];
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int b = 0; b < TB; ++b) acc[t][b] = floatx4{0.f, 0.f, 0.f, 0.f};

  // Per-channel int8: codes of three K steps live in registers (a static ring: the loop
  // is unrolled by three), so while step ks is multiplied the loads of steps ks + 1 and
  // ks + 2 are in flight.  Group-128 formats: one step ahead (the deeper ring costs
  // their 4-token-block variants half their occupancy; measured slower for uint4).  x
  // goes through the LDS double buffer one step ahead.
  constexpr int kAhead = FMT == WQ_FMT_W8_PC ? 2 : 1;
  uint4 c1[RT][CH], c2[RT][CH];
  auto load_codes = [&](uint4 (*c)[CH], int ks) {
    const int kc = min(ks, ks1 - 1);  // past the range: reload the last step (harmless)
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int j = 0; j < CH; ++j) c[t][j] = load_stream16(code_ptr(t, j, kc));
  };
  if (ks0 < ks1) {
    u32x4 xr[XJ];
    xload(xr, ks0);
    load_codes(cw, ks0);
    if constexpr (kAhead == 2) load_codes(c1, ks0 + 1);
    xstore(xr, 0);
    __syncthreads();
  }
  auto step = [&](uint4 (*cur)[CH], uint4 (*fut)[CH], int ks) {
    const int buf = (ks - ks0) & 1;
    const int kn = min(ks + 1, ks1 - 1);
    u32x4 xr[XJ];
    xload(xr, kn);
    load_codes(fut, ks + kAhead);
    const uint8_t* xb = xs[buf];
    transpose(cur);
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      floatx4 part_acc[TB];
#pragma unroll
      for (int b = 0; b < TB; ++b) part_acc[b] = kGrouped ? floatx4{0.f, 0.f, 0.f, 0.f} : acc[t][b];
      if constexpr (!kW4) {
#pragma unroll
        for (int j = 0; j < CH; ++j) {
          const bf16x8_t w0 = __builtin_bit_cast(bf16x8_t, i8x16_to_bf16_lo(cur[t][j]));
          const bf16x8_t w1 = __builtin_bit_cast(bf16x8_t, i8x16_to_bf16_hi(cur[t][j]));
#pragma unroll
          for (int b = 0; b < TB; ++b) {
            const uint8_t* xrow = xb + (16 * b + r16) * SK_XP + 128 * j + 32 * c4;
            const bf16x8_t a0 = *reinterpret_cast<const bf16x8_t*>(xrow);
            const bf16x8_t a1 = *reinterpret_cast<const bf16x8_t*>(xrow + 16);
            part_acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, w0, part_acc[b], 0, 0, 0);
            part_acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, w1, part_acc[b], 0, 0, 0);
          }
        }
      } else {
        const int n = nrow[t];
        const uint8_t zb = zeros[(((size_t)(n / kGemvTileRows) * G + ks) * kGemvTileRows + n % kGemvTileRows) / 2];
        const float z = (float)((zb >> ((n & 1) * 4)) & 0xFu);
        const uint32_t wd[4] = {cur[t][0].x, cur[t][0].y, cur[t][0].z, cur[t][0].w};
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
          const bf16x8_t wv = __builtin_bit_cast(bf16x8_t, w4_word_to_bf16(wd[s2], z));
#pragma unroll
          for (int b = 0; b < TB; ++b) {
            const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(xb + (16 * b + r16) * SK_XP + 64 * c4 + 16 * s2);
            part_acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, wv, part_acc[b], 0, 0, 0);
          }
        }
      }
      if constexpr (kGrouped) {
        const float sc = gscale(nrow[t], ks);
#pragma unroll
        for (int b = 0; b < TB; ++b)
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[t][b][q] = fmaf(sc, part_acc[b][q], acc[t][b][q]);
      } else {
#pragma unroll
        for (int b = 0; b < TB; ++b) acc[t][b] = part_acc[b];
      }
    }
    xstore(xr, buf ^ 1);  // that buffer was last read before the previous barrier
    __syncthreads();
  };
  // ring: step ks multiplies the buffer loaded two steps earlier and loads ks + 2 into
  // the one step ks - 1 has finished with
  if constexpr (kAhead == 2) {
    int ks = ks0;
    for (; ks + 3 <= ks1; ks += 3) {
      step(cw, c2, ks);
      step(c1, cw, ks + 1);
      step(c2, c1, ks + 2);
    }
    if (ks < ks1) step(cw, c2, ks);
    if (ks + 1 < ks1) step(c1, cw, ks + 1);
  } else {
    for (int ks = ks0; ks < ks1; ++ks) {
      step(cw, c1, ks);
#pragma unroll
      for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int j = 0; j < CH; ++j) cw[t][j] = c1[t][j];
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---- epilogue: lane holds D[token 4 c4 + q][weight row r16] of each 16 x 16 block
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const int n = n0 + wave * 32 + t * 16 + r16;
    if (n >= N) continue;
    const float sc = (S == 1 && !kGrouped) ? bf16_to_f32(scales[n]) : 1.f;
#pragma unroll
    for (int b = 0; b < TB; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = 16 * b + 4 * c4 + q;
        if (m >= M) continue;
        if (S == 1)
          y[(size_t)m * N + n] = f32_to_out<false>(with_res<false>(sc * acc[t][b][q], res, (size_t)m * N + n));
        else
          part[((size_t)blockIdx.y * M + m) * N + n] = acc[t][b][q];
      }
  }
}

// Skinny GEMM for M <= 16 (one token block): the x fragments are small enough to come
// straight from memory (x stays in L2), so every wave streams on its own -- no LDS
// staging of x, no barrier -- with the next steps' codes and x in flight while the
// current step's MFMAs run.  Same operand mapping, K order and epilogue as
// gemm_skinny_kernel.  (With two token blocks each wave's x reads double and the LDS-
// staged kernel wins.)
template <int FMT, int TB>
__global__ __launch_bounds__(256) void gemm_skinny_direct_kernel(const uint8_t* __restrict__ qw,
                                                                  const uint16_t* __restrict__ scales,
                                                                  const uint8_t* __restrict__ zeros,
                                                                  const uint16_t* __restrict__ x,
                                                                  uint16_t* y,
                                                                  float* __restrict__ part, int M, int K,
                                                                  int N, int S, const uint16_t* res) {
  constexpr bool kW4 = FMT == WQ_FMT_W4_G128, kGrouped = FMT != WQ_FMT_W8_PC;
  constexpr int RT = 2;              // 16-row tiles per wave
  constexpr int CH = kW4 ? 1 : 2;    // 16-byte code chunks per lane, tile and step
  constexpr int NX = 4;              // x fragments per token block and step (one per MFMA k slice)
  constexpr int kTrPitch = SK_STEP + 16;  // LDS pitch of a transposed code row (bytes, padded)
  __shared__ __attribute__((aligned(16))) uint8_t trs[4][kW4 ? 1 : RT * 16 * kTrPitch];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, c4 = lane >> 4;
  const int n0 = blockIdx.x * SK_ROWS;
  const int KS = K / SK_STEP, G = K / kGroup;
  const int ks0 = (int)((int64_t)KS * blockIdx.y / S), ks1 = (int)((int64_t)KS * (blockIdx.y + 1) / S);
  const int64_t row_bytes = kW4 ? K / 2 : K;

  int nrow[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) nrow[t] = min(n0 + wave * 32 + t * 16 + r16, N - 1);
  // gfx950 code addressing per 16-row tile, split into wave-uniform parts (tile base,
  // rows in the tile) and the lane's row; a step never crosses a 1 KB slice.
  const int wu = __builtin_amdgcn_readfirstlane(wave);
  const int T = (N + kGemvTileRows - 1) / kGemvTileRows;
  const uint8_t* tbase[RT];
  int tnr[RT], trow[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const int ti = min((n0 + wu * 32 + t * 16) / kGemvTileRows, T - 1);
    tnr[t] = min(kGemvTileRows, N - ti * kGemvTileRows);
    tbase[t] = qw + (size_t)ti * kGemvTileRows * row_bytes;
    trow[t] = min(r16, tnr[t] - 1);
  }
  const uint16_t* xrow[TB];
#pragma unroll
  for (int b = 0; b < TB; ++b) xrow[b] = x + (size_t)min(16 * b + r16, M - 1) * K;
  // k offset (elements) of x fragment i within a step: W8 i = 2 j + s -> 64 j + 16 c + 8 s;
  // W4 i = s -> 32 c + 8 s.
  auto xoff = [&](int i) { return kW4 ? 32 * c4 + 8 * i : 64 * (i >> 1) + 16 * c4 + 8 * (i & 1); };
  constexpr int kStepBytes = kW4 ? SK_STEP / 2 : SK_STEP;
  auto load_codes = [&](u32x4 (*dst)[CH], int ks) {
    const int64_t b0 = (int64_t)ks * kStepBytes;
    const int64_t sl = b0 / kSliceBytes;
    const int w = (int)min((int64_t)kSliceBytes, row_bytes - sl * kSliceBytes);
    const int jb = (int)(b0 - sl * kSliceBytes) + 16 * c4;
    if constexpr (kW4) {
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const uint4 v = load_stream16(tbase[t] + (size_t)tnr[t] * kSliceBytes * sl + trow[t] * w + jb);
        dst[t][0] = u32x4{v.x, v.y, v.z, v.w};
      }
    } else {
      // W8: a step is 16 rows x 128 bytes; lane l loads row l / 8 + 8 i, chunk l % 8, so
      // each load instruction covers eight whole 128-byte lines (the fragment layout,
      // 16 rows x 64 bytes per instruction, would fetch half lines).  step() moves the
      // chunks into the fragment layout through this wave's LDS.
      const int jl = (int)(b0 - sl * kSliceBytes) + 16 * (lane & 7);
#pragma unroll
      for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int i = 0; i < CH; ++i) {
          const int rr = min((lane >> 3) + 8 * i, tnr[t] - 1);
          const uint4 v = load_stream16(tbase[t] + (size_t)tnr[t] * kSliceBytes * sl + rr * w + jl);
          dst[t][i] = u32x4{v.x, v.y, v.z, v.w};
        }
    }
  };
  auto load_x = [&](bf16x8_t (*dst)[NX], int ks) {
#pragma unroll
    for (int b = 0; b < TB; ++b)
#pragma unroll
      for (int i = 0; i < NX; ++i) dst[b][i] = *reinterpret_cast<const bf16x8_t*>(xrow[b] + ks * SK_STEP + xoff(i));
  };
  auto gscale = [&](int n, int g) -> float {
    const uint16_t sb = scales[((size_t)(n / kGemvTileRows) * G + g) * kGemvTileRows + n % kGemvTileRows];
    return (FMT == WQ_FMT_W8_G128) ? bf16_to_f32(sb) : f16_to_f32(sb);
  };

  floatx4 acc[RT][TB];
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int b = 0; b < TB; ++b) acc[t][b] = floatx4{0.f, 0.f, 0.f, 0.f};

  // Three register sets with fixed roles, so no set is copied (a copy would wait for
  // its loads): while set s is multiplied, the sets for the next two steps are in
  // flight.
  auto step = [&](const u32x4 (*ld)[CH], const bf16x8_t (*xf_)[NX], int ks) {
    u32x4 cw_[RT][CH];
    if constexpr (kW4) {
#pragma unroll
      for (int t = 0; t < RT; ++t) cw_[t][0] = ld[t][0];
    } else {
      // row-major [row][128 bytes] (pitch kTrPitch) -> lane l gets row l % 16, chunk
      // 4 j + l / 16.  One wave's own region: LDS keeps a wave's accesses in order.
      uint8_t* tw = trs[wave];
#pragma unroll
      for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int i = 0; i < CH; ++i)
          *reinterpret_cast<u32x4*>(tw + (t * 16 + (lane >> 3) + 8 * i) * kTrPitch + 16 * (lane & 7)) = ld[t][i];
#pragma unroll
      for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int j = 0; j < CH; ++j)
          cw_[t][j] = *reinterpret_cast<const u32x4*>(tw + (t * 16 + r16) * kTrPitch + 16 * (4 * j + c4));
    }
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      floatx4 pa[TB];
#pragma unroll
      for (int b = 0; b < TB; ++b) pa[b] = kGrouped ? floatx4{0.f, 0.f, 0.f, 0.f} : acc[t][b];
      if constexpr (!kW4) {
#pragma unroll
        for (int j = 0; j < CH; ++j) {
          const uint4 c = make_uint4(cw_[t][j].x, cw_[t][j].y, cw_[t][j].z, cw_[t][j].w);
          const bf16x8_t w0 = __builtin_bit_cast(bf16x8_t, i8x16_to_bf16_lo(c));
          const bf16x8_t w1 = __builtin_bit_cast(bf16x8_t, i8x16_to_bf16_hi(c));
#pragma unroll
          for (int b = 0; b < TB; ++b) {
            pa[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xf_[b][2 * j], w0, pa[b], 0, 0, 0);
            pa[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xf_[b][2 * j + 1], w1, pa[b], 0, 0, 0);
          }
        }
      } else {
        const int n = nrow[t];
        const uint8_t zb = zeros[(((size_t)(n / kGemvTileRows) * G + ks) * kGemvTileRows + n % kGemvTileRows) / 2];
        const float z = (float)((zb >> ((n & 1) * 4)) & 0xFu);
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
          const bf16x8_t wv = __builtin_bit_cast(bf16x8_t, w4_word_to_bf16(cw_[t][0][s2], z));
#pragma unroll
          for (int b = 0; b < TB; ++b)
            pa[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xf_[b][s2], wv, pa[b], 0, 0, 0);
        }
      }
      if constexpr (kGrouped) {
        const float sc = gscale(nrow[t], ks);
#pragma unroll
        for (int b = 0; b < TB; ++b)
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[t][b][q] = fmaf(sc, pa[b][q], acc[t][b][q]);
      } else {
#pragma unroll
        for (int b = 0; b < TB; ++b) acc[t][b] = pa[b];
      }
    }
  };
  u32x4 ca[RT][CH], cb[RT][CH], cc[RT][CH];
  bf16x8_t xa[TB][NX], xb[TB][NX], xc[TB][NX];
  auto last = [&](int k) { return min(k, ks1 - 1); };  // past the end: reload the last step
  if (ks0 < ks1) {
    load_codes(ca, ks0);
    load_x(xa, ks0);
    load_codes(cb, last(ks0 + 1));
    load_x(xb, last(ks0 + 1));
  }
  for (int ks = ks0; ks < ks1; ks += 3) {
    load_codes(cc, last(ks + 2));
    load_x(xc, last(ks + 2));
    step(ca, xa, ks);
    if (ks + 1 >= ks1) break;
    load_codes(ca, last(ks + 3));
    load_x(xa, last(ks + 3));
    step(cb, xb, ks + 1);
    if (ks + 2 >= ks1) break;
    load_codes(cb, last(ks + 4));
    load_x(xb, last(ks + 4));
    step(cc, xc, ks + 2);
  }

#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const int n = n0 + wave * 32 + t * 16 + r16;
    if (n >= N) continue;
    const float sc = (S == 1 && !kGrouped) ? bf16_to_f32(scales[n]) : 1.f;
#pragma unroll
    for (int b = 0; b < TB; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = 16 * b + 4 * c4 + q;
        if (m >= M) continue;
        if (S == 1)
          y[(size_t)m * N + n] = f32_to_out<false>(with_res<false>(sc * acc[t][b][q], res, (size_t)m * N + n));
        else
          part[((size_t)blockIdx.y * M + m) * N + n] = acc[t][b][q];
      }
  }
}

// y[m][n] = bf16(s[n] * sum_s part[s][m][n]) (per channel) or bf16(sum_s part[s][m][n]),
// the split ranges added in order.
template <bool kPerChannel, bool XF = false>
__global__ __launch_bounds__(256) void gemm_splitk_reduce_kernel(const float* __restrict__ part,
                                                                  const uint16_t* __restrict__ scales,
                                                                  uint16_t* y, int M, int N,
                                                                  int S, const uint16_t* res) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t MN = (int64_t)M * N;
  if (i >= MN) return;
  float v = 0.f;
  for (int s = 0; s < S; ++s) v += part[(int64_t)s * MN + i];
  const float sc = kPerChannel ? bf16_to_f32(scales[i % N]) : 1.f;
  y[i] = f32_to_out<XF>(with_res<XF>(sc * v, res, (size_t)i));
}

// The same sum with four consecutive outputs per thread (M N % 4 == 0): 16-byte partial
// loads, those of four ranges issued together; each output still adds its ranges in
// order from 0, so the results are the scalar kernel's bit for bit.
template <bool kPerChannel, bool XF = false>
__global__ __launch_bounds__(256) void gemm_splitk_reduce4_kernel(const float* __restrict__ part,
                                                                   const uint16_t* __restrict__ scales,
                                                                   uint16_t* y, int M, int N,
                                                                   int S, const uint16_t* res) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;  // this thread's 4-output group
  const int64_t MN = (int64_t)M * N, MN4 = MN / 4;
  if (q >= MN4) return;
  const float4* p4 = reinterpret_cast<const float4*>(part) + q;
  float v[4] = {0.f, 0.f, 0.f, 0.f};
  int s = 0;
  for (; s + 4 <= S; s += 4) {
    float4 a[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) a[j] = p4[(int64_t)(s + j) * MN4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[0] += a[j].x;
      v[1] += a[j].y;
      v[2] += a[j].z;
      v[3] += a[j].w;
    }
  }
  for (; s < S; ++s) {
    const float4 a = p4[(int64_t)s * MN4];
    v[0] += a.x;
    v[1] += a.y;
    v[2] += a.z;
    v[3] += a.w;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t i = 4 * q + j;
    const float sc = kPerChannel ? bf16_to_f32(scales[i % N]) : 1.f;
    y[i] = f32_to_out<XF>(with_res<XF>(sc * v[j], res, (size_t)i));
  }
}

// The split tail tiles of tile 13: y = the ranges' fp32 partials added in range order
// (times the channel scale for per-channel W8).  blockIdx.y: tail tile; a thread takes
// 8 consecutive columns of one row (32 threads per row, 8 rows per block, blockIdx.x:
// the row group).
template <bool kPerChannel, int TM, bool XF = false>
__global__ __launch_bounds__(256) void gemm_tail_reduce_kernel(const float* __restrict__ part,
                                                                const uint16_t* __restrict__ scales,
                                                                uint16_t* y, int M, int N,
                                                                int tail0, int S, const uint16_t* res) {
  const int mblocks = (M + TM - 1) / TM, lin = tail0 + (int)blockIdx.y;
  const int r = (int)blockIdx.x * 8 + (int)(threadIdx.x >> 5), c = 8 * (int)(threadIdx.x & 31);
  const int m = (lin % mblocks) * TM + r, n = (lin / mblocks) * DBN + c;
  if (m >= M || n >= N) return;
  const float* p = part + (size_t)blockIdx.y * S * TM * DBN + r * DBN + c;
  float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < S; ++s) {
    const float4 a = *reinterpret_cast<const float4*>(p + (size_t)s * TM * DBN);
    const float4 b = *reinterpret_cast<const float4*>(p + (size_t)s * TM * DBN + 4);
    v[0] += a.x; v[1] += a.y; v[2] += a.z; v[3] += a.w;
    v[4] += b.x; v[5] += b.y; v[6] += b.z; v[7] += b.w;
  }
  uint16_t o[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float sc = kPerChannel ? bf16_to_f32(scales[min(n + j, N - 1)]) : 1.f;
    o[j] = f32_to_out<XF>(with_res<XF>(sc * v[j], res, (size_t)m * N + min(n + j, N - 1)));
  }
  uint16_t* yo = y + (size_t)m * N + n;
  if (N % 8 == 0) {  // n + 8 <= N and 16-byte aligned
    *reinterpret_cast<uint4*>(yo) = make_uint4(o[0] | (uint32_t)o[1] << 16, o[2] | (uint32_t)o[3] << 16,
                                               o[4] | (uint32_t)o[5] << 16, o[6] | (uint32_t)o[7] << 16);
  } else {
    for (int j = 0; j < 8 && n + j < N; ++j) yo[j] = o[j];
  }
}

template <int FMT>
wq_status launch_skinny(const uint8_t* qw, const uint16_t* sc, const uint8_t* zs, const uint16_t* x,
                        uint16_t* y, float* part, int M, int K, int N, int S, hipStream_t st, const uint16_t* res) {
  const dim3 grid((unsigned)((N + SK_ROWS - 1) / SK_ROWS), (unsigned)S);
  const int TB = (M + 15) / 16;
  // one token block: the direct kernel; two: x through LDS as well (measured at M = 32:
  // 39 us against 57 us for per-channel W8 at (5120, 27648), 53 against 74 for W4)
  if (TB <= 1)
    gemm_skinny_direct_kernel<FMT, 1><<<grid, 256, 0, st>>>(qw, sc, zs, x, y, part, M, K, N, S, res);
  else if (TB <= 2)
    gemm_skinny_kernel<FMT, 2><<<grid, 256, 0, st>>>(qw, sc, zs, x, y, part, M, K, N, S, res);
  else if (TB <= 4)
    gemm_skinny_kernel<FMT, 4><<<grid, 256, 0, st>>>(qw, sc, zs, x, y, part, M, K, N, S, res);
  else
    gemm_skinny_kernel<FMT, 8><<<grid, 256, 0, st>>>(qw, sc, zs, x, y, part, M, K, N, S, res);
  WQ_HIP_CHECK(hipGetLastError());
  if (S > 1) {
    const int64_t MN = (int64_t)M * N;
    gemm_splitk_reduce_kernel<FMT == WQ_FMT_W8_PC>
        <<<(unsigned)((MN + 255) / 256), 256, 0, st>>>(part, sc, y, M, N, S, res);
    WQ_HIP_CHECK(hipGetLastError());
  }
  return WQ_OK;
}

}  // namespace

int gemm_skinny_split(int tile, int64_t M, int64_t N) {
  if (tile < kSkinnyTile0 || tile > kSkinnyTileLast || M > kSkinnyMaxM) return 0;
  const int64_t blocks = (N + SK_ROWS - 1) / SK_ROWS;
  int S = 2 << (tile - kSkinnyTile0);
  // more than kSkinnyMaxBlocks workgroups buys nothing but workspace
  while (S > 1 && (S * M > kSkinnyMaxSplitTokens || blocks * S > 2 * kSkinnyMaxBlocks)) S >>= 1;
  return S;
}

int gemm_dma_split(int fmt, int tile, int64_t M, int64_t N) {
  if ((tile < kDmaSplitTile0 || tile > kDmaSplitTileLast) && tile != kDmaSplit3Tile) return 0;
  const int64_t tm = gemm_big_dma_rows(fmt);
  const int64_t blocks = ((M + tm - 1) / tm) * ((N + DBN - 1) / DBN);
  int S = tile == kDmaSplit3Tile ? 3 : 2 << (tile - kDmaSplitTile0);
  // about two workgroups per CU at most, and a bounded workspace
  while (S > 1 && (blocks * S > 2 * 256 || (int64_t)S * M * N * (int64_t)sizeof(float) > kDmaSplitMaxBytes)) S >>= 1;
  return S;
}

int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return kDefaultCUs;
  int c = cache[dev].load(std::memory_order_relaxed);
  if (c > 0) return c;
  if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c < 1)
    return kDefaultCUs;
  cache[dev].store(c, std::memory_order_relaxed);
  return c;
}

int gemm_dma_tail(int fmt, int64_t M, int64_t N, int* tail0) {
  const int64_t tm = gemm_big_dma_rows(fmt);
  const int64_t total = ((M + tm - 1) / tm) * ((N + DBN - 1) / DBN);
  const int cus = device_cus();
  *tail0 = (int)total;
  const int64_t r = total % cus;
  if (total <= cus || r == 0 || 2 * r > cus) return 1;  // no partial last round to spread
  *tail0 = (int)(total - r);
  return (int)std::min<int64_t>(kDmaTailMaxSplit, cus / r);
}

int gemm_dma64_split(int tile, int64_t M, int64_t N) {
  const int tm = gemm_dma_rows(tile);
  if (tm == 0) return 0;
  const int64_t blocks = ((M + tm - 1) / tm) * ((N + DBN - 1) / DBN);
  int S = tile >= kDma128DeepTile0 ? 8 << (tile - kDma128DeepTile0)
          : tile >= kDma64DeepTile0 ? 8 << (tile - kDma64DeepTile0)
                                    : 1 << (tile - (tm == 64 ? kDma64Tile0 : kDma128Tile0));
  while (S > 1 && (blocks * S > 2 * 256 || (int64_t)S * M * N * (int64_t)sizeof(float) > kDmaSplitMaxBytes)) S >>= 1;
  return S;
}

int gemm_mma_split(int tile, int64_t M, int64_t K) {
  if (tile < kMmaTile0 || tile > kMmaTileLast || M > kMmaTokens) return 0;
  return tile == kMmaTileLast && (K + kGroup - 1) / kGroup >= 2 ? 2 : 1;
}

size_t gemm_workspace_bytes(int fmt, int64_t N, int64_t M, int tile) {
  if (tile >= kMmaTile0 && tile <= kMmaTileLast) {
    const int S = gemm_mma_split(tile, M, 0x7FFFFFFF);
    return S > 1 ? (size_t)S * (size_t)M * (size_t)N * sizeof(float) : 0;
  }
  if (gemm_dma_rows(tile) != 0) {
    const int S = gemm_dma64_split(tile, M, N);
    return S > 1 ? (size_t)S * (size_t)M * (size_t)N * sizeof(float) : 0;
  }
  if (tile == kDmaTailTile) {
    int tail0 = 0;
    const int S = gemm_dma_tail(fmt, M, N, &tail0);
    const int64_t tm = gemm_big_dma_rows(fmt);
    const int64_t total = ((M + tm - 1) / tm) * ((N + DBN - 1) / DBN);
    return S > 1 ? (size_t)S * (size_t)(total - tail0) * tm * DBN * sizeof(float) : 0;
  }
  const int S = tile >= kDmaSplitTile0 ? gemm_dma_split(fmt, tile, M, N) : gemm_skinny_split(tile, M, N);
  return S > 1 ? (size_t)S * (size_t)M * (size_t)N * sizeof(float) : 0;
}

static size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }

size_t gemm_workspace_full_bytes(int fmt, int64_t K, int64_t N, int64_t M, int tile) {
  const size_t need = gemm_workspace_bytes(fmt, N, M, tile);
  const bool dma = tile >= 9 && (tile < kMmaTile0 || tile >= kDmaSplit3Tile);
  if (fmt == WQ_FMT_W8_PC || !dma || K % DBK != 0 || M * K >= (int64_t(1) << 31)) return need;
  return round256(round256(need) + (size_t)M * (size_t)K * 2) + (size_t)M * sizeof(float);
}

// The fp16 copy of x (rows scaled) and the row scales' inverses after part_bytes of
// partials, when the workspace has room for both: launches x_to_f16_rows_kernel and sets
// *xh and *xinv, else leaves them NULL (the tiles then convert x in LDS).
static hipError_t x_to_f16_rows(const uint16_t* x, int64_t M, int K, void* ws, size_t ws_bytes, size_t part_bytes,
                                uint16_t** xh, float** xinv, hipStream_t s) {
  const size_t xh_off = round256(part_bytes), xi_off = round256(xh_off + (size_t)M * K * 2);
  if (!ws || ws_bytes < xi_off + (size_t)M * sizeof(float) || ((uintptr_t)ws + xh_off) % 16 != 0) return hipSuccess;
  *xh = (uint16_t*)((uint8_t*)ws + xh_off);
  *xinv = (float*)((uint8_t*)ws + xi_off);
  // threads: a 16-byte chunk each (whole waves, at most 1024) while the rows are few; from
  // 256 rows on, 256 per row (measured on MI355X at M = 2048, K = 5120: the wide rows took
  // 15 us against about 10 us with 256 threads)
  const int64_t per_row = std::min<int64_t>(M >= 256 ? 256 : 1024, ((K / 8 + 63) / 64) * 64);
  const int thr = (int)std::max<int64_t>(64, per_row);
  x_to_f16_rows_kernel<<<(unsigned)M, thr, 0, s>>>(x, *xh, *xinv, K);
  return hipGetLastError();
}

// The grouped LDS-DMA kernel for a format family, x-tile height and group size, fed by
// the fp16 copy of x when there is one (xh), else converting x itself.
template <int F, int TMV, int GS>
static void g_dma_launch(dim3 grid, hipStream_t s, const uint8_t* qw, const uint16_t* sc, const uint8_t* zs,
                         const uint16_t* x, const uint16_t* xh, const float* xinv, uint16_t* y, float* part, int M,
                         int K, int N, int tail0, int tailS, bool xf, const uint16_t* res) {
  if (xf)  // fp16 activations: x is the fp16 operand
    gemm_dma_g128_kernel<F, 1, 8, true, TMV, GS, true>
        <<<grid, 512, 0, s>>>(qw, sc, zs, x, x, nullptr, y, part, M, K, N, tail0, tailS, res);
  else if (xh)
    gemm_dma_g128_kernel<F, 1, 8, true, TMV, GS>
        <<<grid, 512, 0, s>>>(qw, sc, zs, x, xh, xinv, y, part, M, K, N, tail0, tailS, res);
  else
    gemm_dma_g128_kernel<F, 1, 8, false, TMV, GS>
        <<<grid, 512, 0, s>>>(qw, sc, zs, x, x, nullptr, y, part, M, K, N, tail0, tailS, res);
}
template <int F, int TMV>
static void g_dma_launch_gs(int gs, dim3 grid, hipStream_t s, const uint8_t* qw, const uint16_t* sc,
                            const uint8_t* zs, const uint16_t* x, const uint16_t* xh, const float* xinv, uint16_t* y,
                            float* part, int M, int K, int N, int tail0, int tailS, bool xf, const uint16_t* res) {
  if (gs == 32) g_dma_launch<F, TMV, 32>(grid, s, qw, sc, zs, x, xh, xinv, y, part, M, K, N, tail0, tailS, xf, res);
  else if (gs == 64) g_dma_launch<F, TMV, 64>(grid, s, qw, sc, zs, x, xh, xinv, y, part, M, K, N, tail0, tailS, xf, res);
  else g_dma_launch<F, TMV, kGroup>(grid, s, qw, sc, zs, x, xh, xinv, y, part, M, K, N, tail0, tailS, xf, res);
}
static void g_dma_dispatch(int fmt, int tm, dim3 grid, hipStream_t s, const uint8_t* qw, const uint16_t* sc,
                           const uint8_t* zs, const uint16_t* x, const uint16_t* xh, const float* xinv, uint16_t* y,
                           float* part, int M, int K, int N, int tail0, int tailS, bool xf, const uint16_t* res) {
  const int gs = meta_group(fmt);
  if (family(fmt) == WQ_FMT_W4_G128) {
    if (tm == 64)
      g_dma_launch_gs<WQ_FMT_W4_G128, 64>(gs, grid, s, qw, sc, zs, x, xh, xinv, y, part, M, K, N, tail0, tailS, xf, res);
    else
      g_dma_launch_gs<WQ_FMT_W4_G128, 128>(gs, grid, s, qw, sc, zs, x, xh, xinv, y, part, M, K, N, tail0, tailS, xf, res);
  } else {
    if (tm == 64)
      g_dma_launch_gs<WQ_FMT_W8_G128, 64>(gs, grid, s, qw, sc, zs, x, xh, xinv, y, part, M, K, N, tail0, tailS, xf, res);
    else
      g_dma_launch_gs<WQ_FMT_W8_G128, 128>(gs, grid, s, qw, sc, zs, x, xh, xinv, y, part, M, K, N, tail0, tailS, xf, res);
  }
}
// the split-K reduction of the GEMM tiles, with the output type of the call
static void splitk_reduce(bool pc, bool xf, const float* part, const uint16_t* sc, uint16_t* y, int64_t M, int N,
                          int S, hipStream_t s, const uint16_t* res) {
  const int64_t MN = M * N;
  if (MN % 4 == 0) {  // four outputs per thread (the partials are 16-byte aligned: ws is 256-byte aligned)
    const unsigned b4 = (unsigned)((MN / 4 + 255) / 256);
    if (pc && xf) gemm_splitk_reduce4_kernel<true, true><<<b4, 256, 0, s>>>(part, sc, y, (int)M, N, S, res);
    else if (pc) gemm_splitk_reduce4_kernel<true><<<b4, 256, 0, s>>>(part, sc, y, (int)M, N, S, res);
    else if (xf) gemm_splitk_reduce4_kernel<false, true><<<b4, 256, 0, s>>>(part, sc, y, (int)M, N, S, res);
    else gemm_splitk_reduce4_kernel<false><<<b4, 256, 0, s>>>(part, sc, y, (int)M, N, S, res);
    return;
  }
  const unsigned blocks = (unsigned)((MN + 255) / 256);
  if (pc && xf) gemm_splitk_reduce_kernel<true, true><<<blocks, 256, 0, s>>>(part, sc, y, (int)M, N, S, res);
  else if (pc) gemm_splitk_reduce_kernel<true><<<blocks, 256, 0, s>>>(part, sc, y, (int)M, N, S, res);
  else if (xf) gemm_splitk_reduce_kernel<false, true><<<blocks, 256, 0, s>>>(part, sc, y, (int)M, N, S, res);
  else gemm_splitk_reduce_kernel<false><<<blocks, 256, 0, s>>>(part, sc, y, (int)M, N, S, res);
}

wq_status launch_gemm(const wq_weight* w, const uint16_t* x, int64_t M, uint16_t* y, int tile,
                      void* ws, size_t ws_bytes, hipStream_t s, bool xf, const uint16_t* res) {
  const int K = (int)w->K, N = (int)w->N;
  if (M > 65535LL * BM) return fail(WQ_ERR_UNSUPPORTED, "wq_gemm: M too large");
  const uint8_t* qw = (const uint8_t*)w->qweight;
  const uint16_t* sc = (const uint16_t*)w->scales;
  const uint8_t* zs = (const uint8_t*)w->zeros;
  if (w->fmt == WQ_FMT_W4_PC) return fail(WQ_ERR_UNSUPPORTED, "wq_gemm: per-channel W4 runs through its compute view");
  if (xf) tile = act_tile(w->fmt, tile);  // the kernels with an fp16-activation form
  else if (small_group(w->fmt)) tile = small_group_tile(tile);
  if (tile >= kMmaTile0 && tile <= kMmaTileLast) {
    // 8..16 tokens: the matrix-core GEMV kernel (one 16-token A operand)
    int S = gemm_mma_split(tile, M, K);
    if (S > 0) {
      if (S > 1 && (!ws || ws_bytes < gemm_workspace_bytes(w->fmt, N, M, tile))) S = 1;  // no room for partials
      const int nb = tile == kMmaTile0 + 1 ? 2 : tile == kMmaTile0 + 2 ? 4 : 1;
      const int rows = (16 * nb) | kGemvMfma;
      return launch_gemv(w, x, (int)M, y, S, gemv_default_waves(K, N, w->fmt, (int)M, S, rows), rows, ws, s, false, res);
    }
    tile = K % DBK == 0 ? kDma64Tile0 : 2;  // more tokens than one A operand holds
  }
  if (tile >= kSkinnyTile0 && tile <= kSkinnyTileLast) {
    int S = gemm_skinny_split(tile, M, N);
    if (S > 0 && K % SK_STEP == 0 && (int64_t)M * K < (int64_t(1) << 31)) {
      if (S > 1 && (!ws || ws_bytes < gemm_workspace_bytes(w->fmt, N, M, tile))) S = 1;  // no room for partials
      float* part = (float*)ws;
      switch (w->fmt) {
        case WQ_FMT_W8_PC: return launch_skinny<WQ_FMT_W8_PC>(qw, sc, zs, x, y, part, (int)M, K, N, S, s, res);
        case WQ_FMT_W8_G128: return launch_skinny<WQ_FMT_W8_G128>(qw, sc, zs, x, y, part, (int)M, K, N, S, s, res);
        case WQ_FMT_W4_G128: return launch_skinny<WQ_FMT_W4_G128>(qw, sc, zs, x, y, part, (int)M, K, N, S, s, res);
        default: return fail(WQ_ERR_UNSUPPORTED, "wq_gemm: unknown format");
      }
    }
    tile = 2;  // shape outside the skinny kernel's range
  }
  // LDS-DMA tiles: 3, 4 and 9 (per-channel W8; for group-128 only the 8-wave tile 9 --
  // the 4-wave layouts would spill its registers -- and tiles 3 and 4 take tile 1), and
  // 10..12: tile 9 with split-K 2, 4, 8 (fp32 partials in the workspace, added in
  // range order by a second kernel; split 1 when the workspace is too small)
  const bool pc = w->fmt == WQ_FMT_W8_PC;
  const int tm = gemm_dma_rows(tile);
  if (tm != 0 && K % DBK == 0 && M * K < (int64_t(1) << 31)) {
    // 64- and 128-row LDS-DMA tiles, split-K 1 / 2 / 4 (8 / 16 for 25 / 26 and 27 / 28) over gridDim.y
    const int64_t total = ((M + tm - 1) / tm) * ((N + DBN - 1) / DBN);
    int S = gemm_dma64_split(tile, M, N);
    if (S > 1 && (!ws || ws_bytes < gemm_workspace_bytes(w->fmt, N, M, tile))) S = 1;
    S = std::min(S, K / (DBK * (pc ? 1 : 2)));
    const dim3 grid((unsigned)(8 * ((total + 7) / 8)), (unsigned)S);
    float* part = (float*)ws;
    if (pc) {
      if (tm == 64 && xf)
        gemm_dma64_w8pc_kernel<64, true><<<grid, 512, 0, s>>>(qw, sc, x, y, part, (int)M, K, N, (int)total, 1, res);
      else if (tm == 64)
        gemm_dma64_w8pc_kernel<64><<<grid, 512, 0, s>>>(qw, sc, x, y, part, (int)M, K, N, (int)total, 1, res);
      else if (xf)
        gemm_dma64_w8pc_kernel<128, true><<<grid, 512, 0, s>>>(qw, sc, x, y, part, (int)M, K, N, (int)total, 1, res);
      else
        gemm_dma64_w8pc_kernel<128><<<grid, 512, 0, s>>>(qw, sc, x, y, part, (int)M, K, N, (int)total, 1, res);
    } else {
      uint16_t* xh = nullptr;
      float* xinv = nullptr;
      if (!xf)
        WQ_HIP_CHECK(x_to_f16_rows(x, M, K, ws, ws_bytes, S > 1 ? (size_t)S * M * N * sizeof(float) : 0, &xh,
                                   &xinv, s));
      g_dma_dispatch(w->fmt, tm, grid, s, qw, sc, zs, x, xh, xinv, y, part, (int)M, K, N, (int)total, 1, xf, res);
    }
    WQ_HIP_CHECK(hipGetLastError());
    if (S > 1) {
      splitk_reduce(pc, xf, part, sc, y, M, N, S, s, res);
      WQ_HIP_CHECK(hipGetLastError());
    }
    return WQ_OK;
  }
  if (tm != 0) tile = 1;  // shapes outside the LDS-DMA tiles
  const bool dma_tile = tile == 3 || tile == 4 || tile >= 9;
  if (dma_tile && (pc || tile >= 9) && K % DBK == 0 && M * K < (int64_t(1) << 31)) {
    // per-channel W8: 256 x 256 tiles; group-128: 128 x 256 tiles (the exact kernel's
    // second accumulator set)
    const int btm = gemm_big_dma_rows(w->fmt);
    const int64_t total = ((M + btm - 1) / btm) * ((N + DBN - 1) / DBN);
    const int kcap = K / (DBK * (pc ? 1 : 2));  // at least one step (group) per K range
    int S = 1, tail0 = (int)total, tailS = 1;
    if (tile == kDmaTailTile) {
      tailS = std::min(gemm_dma_tail(w->fmt, M, N, &tail0), kcap);
      if (tailS <= 1 || !ws || ws_bytes < gemm_workspace_bytes(w->fmt, N, M, tile)) {
        tailS = 1;
        tail0 = (int)total;
      }
    } else if (tile >= kDmaSplitTile0) {
      S = gemm_dma_split(w->fmt, tile, M, N);
      if (S > 1 && (!ws || ws_bytes < gemm_workspace_bytes(w->fmt, N, M, tile))) S = 1;
      S = std::min(S, kcap);
    }
    const int64_t ntail = total - tail0;
    const unsigned blocks = (unsigned)(8 * ((tail0 + 7) / 8) + 8 * ((tailS * ntail + 7) / 8));
    const dim3 grid(blocks, (unsigned)S);
    float* part = (float*)ws;
    const size_t part_bytes = tailS > 1 ? (size_t)tailS * ntail * btm * DBN * sizeof(float)
                                        : (S > 1 ? (size_t)S * M * N * sizeof(float) : 0);
    if (pc) {
      if (xf)  // (tiles 3 and 4 run as 9 for fp16 activations)
        gemm_dma_w8pc_kernel<2, 4, true><<<grid, 512, 0, s>>>(qw, sc, x, y, part, (int)M, K, N, tail0, tailS, res);
      else if (tile == 3)
        gemm_dma_w8pc_kernel<2, 2><<<grid, 256, 0, s>>>(qw, sc, x, y, part, (int)M, K, N, tail0, tailS, res);
      else if (tile == 4)
        gemm_dma_w8pc_kernel<1, 4><<<grid, 256, 0, s>>>(qw, sc, x, y, part, (int)M, K, N, tail0, tailS, res);
      else
        gemm_dma_w8pc_kernel<2, 4><<<grid, 512, 0, s>>>(qw, sc, x, y, part, (int)M, K, N, tail0, tailS, res);
    } else {
      // x in fp16 (rows scaled) after the partials when the workspace has room for it
      uint16_t* xh = nullptr;
      float* xinv = nullptr;
      if (!xf) WQ_HIP_CHECK(x_to_f16_rows(x, M, K, ws, ws_bytes, part_bytes, &xh, &xinv, s));
      g_dma_dispatch(w->fmt, 128, grid, s, qw, sc, zs, x, xh, xinv, y, part, (int)M, K, N, tail0, tailS, xf, res);
    }
    WQ_HIP_CHECK(hipGetLastError());
    if (S > 1) {
      splitk_reduce(pc, xf, part, sc, y, M, N, S, s, res);
      WQ_HIP_CHECK(hipGetLastError());
    }
    if (tailS > 1) {
      const dim3 rg((unsigned)(btm / 8), (unsigned)ntail);
      if (pc && xf)
        gemm_tail_reduce_kernel<true, 256, true><<<rg, 256, 0, s>>>(part, sc, y, (int)M, N, tail0, tailS, res);
      else if (pc)
        gemm_tail_reduce_kernel<true, 256><<<rg, 256, 0, s>>>(part, sc, y, (int)M, N, tail0, tailS, res);
      else if (xf)
        gemm_tail_reduce_kernel<false, 128, true><<<rg, 256, 0, s>>>(part, sc, y, (int)M, N, tail0, tailS, res);
      else
        gemm_tail_reduce_kernel<false, 128><<<rg, 256, 0, s>>>(part, sc, y, (int)M, N, tail0, tailS, res);
      WQ_HIP_CHECK(hipGetLastError());
    }
    return WQ_OK;
  }
  if (dma_tile) tile = 1;
  if (tile == 1 && !small_group(w->fmt) && !xf) {  // (groups of 32 and 64 and fp16 x take tile 2's kernel)
    const int bn = w->fmt == WQ_FMT_W8_PC ? Big<WQ_FMT_W8_PC>::BN : Big<WQ_FMT_W8_G128>::BN;
    const int64_t total = ((M + BM2 - 1) / BM2) * ((N + bn - 1) / bn);
    const unsigned blocks = (unsigned)(8 * ((total + 7) / 8));
    switch (w->fmt) {
      case WQ_FMT_W8_PC:
        gemm_big_kernel<WQ_FMT_W8_PC><<<blocks, 256, 0, s>>>(qw, sc, zs, x, y, (int)M, K, N, res);
        break;
      case WQ_FMT_W8_G128:
        gemm_big_kernel<WQ_FMT_W8_G128><<<blocks, 256, 0, s>>>(qw, sc, zs, x, y, (int)M, K, N, res);
        break;
      case WQ_FMT_W4_G128:
        gemm_big_kernel<WQ_FMT_W4_G128><<<blocks, 256, 0, s>>>(qw, sc, zs, x, y, (int)M, K, N, res);
        break;
      default:
        return fail(WQ_ERR_UNSUPPORTED, "wq_gemm: unknown format");
    }
    WQ_HIP_CHECK(hipGetLastError());
    return WQ_OK;
  }
  dim3 grid((N + BN - 1) / BN, (unsigned)((M + BM - 1) / BM));
  const int gshift = meta_group(w->fmt) == 32 ? 5 : meta_group(w->fmt) == 64 ? 6 : 7;
  switch (family(w->fmt)) {
    case WQ_FMT_W8_PC:
      if (xf) gemm_kernel<WQ_FMT_W8_PC, true><<<grid, 256, 0, s>>>(qw, sc, zs, x, y, (int)M, K, N, gshift, res);
      else gemm_kernel<WQ_FMT_W8_PC><<<grid, 256, 0, s>>>(qw, sc, zs, x, y, (int)M, K, N, gshift, res);
      break;
    case WQ_FMT_W8_G128:
      if (xf) gemm_kernel<WQ_FMT_W8_G128, true><<<grid, 256, 0, s>>>(qw, sc, zs, x, y, (int)M, K, N, gshift, res);
      else gemm_kernel<WQ_FMT_W8_G128><<<grid, 256, 0, s>>>(qw, sc, zs, x, y, (int)M, K, N, gshift, res);
      break;
    case WQ_FMT_W4_G128:
      if (xf) gemm_kernel<WQ_FMT_W4_G128, true><<<grid, 256, 0, s>>>(qw, sc, zs, x, y, (int)M, K, N, gshift, res);
      else gemm_kernel<WQ_FMT_W4_G128><<<grid, 256, 0, s>>>(qw, sc, zs, x, y, (int)M, K, N, gshift, res);
      break;
    default:
      return fail(WQ_ERR_UNSUPPORTED, "wq_gemm: unknown format");
  }
  WQ_HIP_CHECK(hipGetLastError());
  return WQ_OK;
}

}  // namespace wq
