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

namespace wq {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
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

// gfx950 int8 codes are u = q + 128; flipping the sign bit gives q.
__device__ __forceinline__ uint4 i8x16_to_bf16_lo(uint4 v) {
  auto cvt = [](uint32_t d) -> uint2 {
    d ^= 0x80808080u;
    return make_uint2(pack_bf16x2((float)(int8_t)(d & 0xFFu), (float)(int8_t)((d >> 8) & 0xFFu)),
                      pack_bf16x2((float)(int8_t)((d >> 16) & 0xFFu), (float)(int8_t)(d >> 24)));
  };
  uint2 a = cvt(v.x), b = cvt(v.y);
  return make_uint4(a.x, a.y, b.x, b.y);
}
__device__ __forceinline__ uint4 i8x16_to_bf16_hi(uint4 v) {
  return i8x16_to_bf16_lo(make_uint4(v.z, v.w, 0, 0));
}

// One gfx950-layout W4 word (8 codes, nibbles q0 q2 q4 q6 q1 q3 q5 q7) -> 8 exact bf16 (q - z).
__device__ __forceinline__ uint4 w4_word_to_bf16(uint32_t w, float z) {
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = (float)((w >> (4 * i)) & 0xFu) - z;
    const float hi = (float)((w >> (16 + 4 * i)) & 0xFu) - z;
    o[i] = pack_bf16x2(lo, hi);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

template <int FMT>
__global__ __launch_bounds__(256) void gemm_kernel(const uint8_t* __restrict__ qw,
                                                     const uint16_t* __restrict__ scales,
                                                     const uint8_t* __restrict__ zeros,
                                                     const uint16_t* __restrict__ x,
                                                     uint16_t* __restrict__ y, int M, int K, int N) {
  __shared__ __attribute__((aligned(16))) uint16_t As[BM * LDA];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[BN * LDA];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
  const int G = K / kGroup;
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
        *reinterpret_cast<uint4*>(&Bs[row * LDA + col]) = i8x16_to_bf16_lo(wb[j]);
        *reinterpret_cast<uint4*>(&Bs[row * LDA + col + 8]) = i8x16_to_bf16_hi(wb[j]);
      }
    } else {
      const int row = tid >> 1, col = (tid & 1) * 32;
      const int n = min(n0 + row, N - 1);
      const int g = k0 / kGroup;
      const uint32_t zb = zeros[(((size_t)(n / kGemvTileRows) * G + g) * kGemvTileRows + n % kGemvTileRows) / 2];
      const float z = (float)((zb >> ((n & 1) * 4)) & 0xFu);
      *reinterpret_cast<uint4*>(&Bs[row * LDA + col + 0]) = w4_word_to_bf16(wb[0].x, z);
      *reinterpret_cast<uint4*>(&Bs[row * LDA + col + 8]) = w4_word_to_bf16(wb[0].y, z);
      *reinterpret_cast<uint4*>(&Bs[row * LDA + col + 16]) = w4_word_to_bf16(wb[0].z, z);
      *reinterpret_cast<uint4*>(&Bs[row * LDA + col + 24]) = w4_word_to_bf16(wb[0].w, z);
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
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          if constexpr (kGrouped)
            tmp[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], tmp[i][j], 0, 0, 0);
          else
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
    }
    if constexpr (kGrouped) {
      if (((k0 + BK) % kGroup) == 0) {
        const int g = k0 / kGroup;
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
        if (m < M) y[(size_t)m * N + n] = __builtin_bit_cast(uint16_t, (__bf16)(s * acc[i][j][a]));
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
                                                           uint16_t* __restrict__ y, int M, int K, int N) {
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
        if (m < M) y[(size_t)m * N + n] = __builtin_bit_cast(uint16_t, (__bf16)(sc * acc[i][j][a]));
      }
  }
}

}  // namespace

wq_status launch_gemm(const wq_weight* w, const uint16_t* x, int64_t M, uint16_t* y, int tile,
                      hipStream_t s) {
  const int K = (int)w->K, N = (int)w->N;
  if (M > 65535LL * BM) return fail(WQ_ERR_UNSUPPORTED, "wq_gemm: M too large");
  const uint8_t* qw = (const uint8_t*)w->qweight;
  const uint16_t* sc = (const uint16_t*)w->scales;
  const uint8_t* zs = (const uint8_t*)w->zeros;
  if (tile == 1) {
    const int bn = w->fmt == WQ_FMT_W8_PC ? Big<WQ_FMT_W8_PC>::BN : Big<WQ_FMT_W8_G128>::BN;
    const int64_t total = ((M + BM2 - 1) / BM2) * ((N + bn - 1) / bn);
    const unsigned blocks = (unsigned)(8 * ((total + 7) / 8));
    switch (w->fmt) {
      case WQ_FMT_W8_PC:
        gemm_big_kernel<WQ_FMT_W8_PC><<<blocks, 256, 0, s>>>(qw, sc, zs, x, y, (int)M, K, N);
        break;
      case WQ_FMT_W8_G128:
        gemm_big_kernel<WQ_FMT_W8_G128><<<blocks, 256, 0, s>>>(qw, sc, zs, x, y, (int)M, K, N);
        break;
      case WQ_FMT_W4_G128:
        gemm_big_kernel<WQ_FMT_W4_G128><<<blocks, 256, 0, s>>>(qw, sc, zs, x, y, (int)M, K, N);
        break;
      default:
        return fail(WQ_ERR_UNSUPPORTED, "wq_gemm: unknown format");
    }
    WQ_HIP_CHECK(hipGetLastError());
    return WQ_OK;
  }
  dim3 grid((N + BN - 1) / BN, (unsigned)((M + BM - 1) / BM));
  switch (w->fmt) {
    case WQ_FMT_W8_PC:
      gemm_kernel<WQ_FMT_W8_PC><<<grid, 256, 0, s>>>(qw, sc, zs, x, y, (int)M, K, N);
      break;
    case WQ_FMT_W8_G128:
      gemm_kernel<WQ_FMT_W8_G128><<<grid, 256, 0, s>>>(qw, sc, zs, x, y, (int)M, K, N);
      break;
    case WQ_FMT_W4_G128:
      gemm_kernel<WQ_FMT_W4_G128><<<grid, 256, 0, s>>>(qw, sc, zs, x, y, (int)M, K, N);
      break;
    default:
      return fail(WQ_ERR_UNSUPPORTED, "wq_gemm: unknown format");
  }
  WQ_HIP_CHECK(hipGetLastError());
  return WQ_OK;
}

}  // namespace wq
