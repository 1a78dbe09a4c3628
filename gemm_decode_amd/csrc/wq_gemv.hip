// Decode GEMV for 1 <= M <= 7 tokens: y[m][n] = sum_k x[m][k] * dequant(W)[n][k].
//
// Design (gfx950, wave64):
//   * A wave owns kGemvRowsPerWave consecutive output rows and one split-K slice.
//     Each lane streams 16-byte chunks of every row (128-bit global loads of
//     packed int8 / int4 codes), so a wave instruction reads 1 KB contiguous of a
//     row; the same x chunk (bf16, from L2/L1) serves all rows of the wave.
//   * Codes are turned into exact bf16 pairs in registers and multiplied with
//     bf16 x pairs by v_dot2 (two MACs, fp32 accumulate):
//       - int8: v_cvt_f32_i32 with a sign-extended byte select, then
//         v_cvt_pk_bf16_f32 (|q| <= 127 is exact in bf16);
//       - uint4 (nibbles interleaved by the gfx950 repack): (word >> 4i) &
//         0x000F000F | 0x43004300 is the bf16 pair (128 + q_2i, 128 + q_2i+1)
//         exactly; the offset is removed per 32-element chunk as
//         (128 + z) * sum(x) before the group scale is applied.
//   * Scales are applied to fp32 partial sums (per row at the end for
//     per-channel W8, per 16/32-element chunk for group-128) so the codes stay
//     exact.
//   * Cross-lane reduction with DPP row operations plus lane reads.
//   * Split-K: each slice writes fp32 partials; the last wave to arrive at a row
//     tile (an atomic counter in the workspace) sums the slices in slice order
//     and writes bf16 y, then resets the counter to zero.
//
// Prior art: the tileInfer README ("Key Optimizations": register-only dequantize
// GEMV with 128-bit loads and warp-shuffle reduction, split-K by its kernel name
// in the project tree) and the Marlin benchmark page (intro: FP32 reduction
// scratch for cross-block partial sums).  Nothing here follows their code.
#include "wq_internal.h"

namespace wq {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int RW = kGemvRowsPerWave;
constexpr int kWaves = 4;                 // waves per block
constexpr size_t kCounterBytes = 256 * 1024;  // counters live at the start of the workspace

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v;
  v.x = (__bf16)lo;
  v.y = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// Four int8 codes of `d` -> two exact bf16 pairs.
__device__ __forceinline__ void i8x4_to_bf16(uint32_t d, uint32_t& p0, uint32_t& p1) {
  const float f0 = (float)(int8_t)(d & 0xFFu);
  const float f1 = (float)(int8_t)((d >> 8) & 0xFFu);
  const float f2 = (float)(int8_t)((d >> 16) & 0xFFu);
  const float f3 = (float)(int8_t)(d >> 24);
  p0 = pack_bf16x2(f0, f1);
  p1 = pack_bf16x2(f2, f3);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ float f16_to_f32(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

__device__ __forceinline__ uint16_t f32_to_bf16(float v) {
  return __builtin_bit_cast(uint16_t, (__bf16)v);  // v_cvt_pk_bf16_f32: nearest even
}

// Sum over the 64 lanes of a wave; the result is returned in every lane.
__device__ __forceinline__ float wave_sum(float v) {
  // within each row of 16 lanes: xor 1, xor 2 (quad permutes), half-row and row mirrors
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false));
  // the four row sums
  const int iv = __builtin_bit_cast(int, v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 48));
  return (r0 + r1) + (r2 + r3);
}

template <int FMT>
struct Fmt;
template <>
struct Fmt<WQ_FMT_W8_PC> {
  static constexpr int kPerChunk = 16;   // k values per 16-byte chunk
  static constexpr int kChunksPerUnit = 1;
};
template <>
struct Fmt<WQ_FMT_W8_G128> {
  static constexpr int kPerChunk = 16;
  static constexpr int kChunksPerUnit = 8;  // one 128-group
};
template <>
struct Fmt<WQ_FMT_W4_G128> {
  static constexpr int kPerChunk = 32;
  static constexpr int kChunksPerUnit = 4;
};

template <int FMT, int M>
__global__ __launch_bounds__(256) void gemv_kernel(const uint8_t* __restrict__ qw,
                                                     const uint16_t* __restrict__ scales,
                                                     const uint8_t* __restrict__ zeros,
                                                     const uint16_t* __restrict__ x,
                                                     uint16_t* __restrict__ y,
                                                     uint32_t* __restrict__ counters,
                                                     float* __restrict__ part, int K, int N,
                                                     int split_k) {
  using F = Fmt<FMT>;
  const int lane = threadIdx.x & 63;
  const int tile = blockIdx.x * kWaves + (threadIdx.x >> 6);  // row tile of this wave
  const int n0 = tile * RW;
  if (n0 >= N) return;  // whole wave leaves together
  const int s = blockIdx.y;

  const int chunks_row = K / F::kPerChunk;
  const int units = chunks_row / F::kChunksPerUnit;
  const int c0 = (int)(((int64_t)s * units) / split_k) * F::kChunksPerUnit;
  const int c1 = (int)(((int64_t)(s + 1) * units) / split_k) * F::kChunksPerUnit;
  const int G = K / kGroup;
  const int Gh = (G + 1) / 2;
  const size_t row_bytes = (FMT == WQ_FMT_W4_G128) ? (size_t)K / 2 : (size_t)K;

  const uint8_t* rowp[RW];
  int rown[RW];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    rown[r] = min(n0 + r, N - 1);
    rowp[r] = qw + (size_t)rown[r] * row_bytes;
  }

  float acc[RW][M];
#pragma unroll
  for (int r = 0; r < RW; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] = 0.f;

#pragma unroll 2
  for (int c = c0 + lane; c < c1; c += 64) {
    uint4 wv[RW];
#pragma unroll
    for (int r = 0; r < RW; ++r) wv[r] = *reinterpret_cast<const uint4*>(rowp[r] + (size_t)c * 16);

    if constexpr (FMT != WQ_FMT_W4_G128) {
      // x chunk: 16 bf16 = 8 pairs per token
      uint32_t xp[M][8];
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const uint4* xs = reinterpret_cast<const uint4*>(x + (size_t)m * K + (size_t)c * 16);
        uint4 a = xs[0], b = xs[1];
        xp[m][0] = a.x; xp[m][1] = a.y; xp[m][2] = a.z; xp[m][3] = a.w;
        xp[m][4] = b.x; xp[m][5] = b.y; xp[m][6] = b.z; xp[m][7] = b.w;
      }
#pragma unroll
      for (int r = 0; r < RW; ++r) {
        uint32_t wp[8];
        i8x4_to_bf16(wv[r].x, wp[0], wp[1]);
        i8x4_to_bf16(wv[r].y, wp[2], wp[3]);
        i8x4_to_bf16(wv[r].z, wp[4], wp[5]);
        i8x4_to_bf16(wv[r].w, wp[6], wp[7]);
        if constexpr (FMT == WQ_FMT_W8_PC) {
#pragma unroll
          for (int m = 0; m < M; ++m)
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[r][m] = dot2(wp[i], xp[m][i], acc[r][m]);
        } else {
          const float sc = bf16_to_f32(scales[(size_t)rown[r] * G + (c >> 3)]);
#pragma unroll
          for (int m = 0; m < M; ++m) {
            float t = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) t = dot2(wp[i], xp[m][i], t);
            acc[r][m] = fmaf(sc, t, acc[r][m]);
          }
        }
      }
    } else {
      // x chunk: 32 bf16 = 16 pairs per token, and its sum
      uint32_t xp[M][16];
      float xsum[M];
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const uint4* xs = reinterpret_cast<const uint4*>(x + (size_t)m * K + (size_t)c * 32);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint4 a = xs[j];
          xp[m][4 * j + 0] = a.x; xp[m][4 * j + 1] = a.y; xp[m][4 * j + 2] = a.z; xp[m][4 * j + 3] = a.w;
        }
        float t = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) t = dot2(xp[m][i], 0x3F803F80u, t);
        xsum[m] = t;
      }
      const int g = c >> 2;
#pragma unroll
      for (int r = 0; r < RW; ++r) {
        const float sc = f16_to_f32(scales[(size_t)rown[r] * G + g]);
        const uint32_t zb = zeros[(size_t)rown[r] * Gh + (g >> 1)];
        const float off = 128.f + (float)((zb >> ((g & 1) * 4)) & 0xFu);
        const uint32_t words[4] = {wv[r].x, wv[r].y, wv[r].z, wv[r].w};
        float t[M];
#pragma unroll
        for (int m = 0; m < M; ++m) t[m] = 0.f;
#pragma unroll
        for (int wi = 0; wi < 4; ++wi) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t p = ((words[wi] >> (4 * i)) & 0x000F000Fu) | 0x43004300u;
#pragma unroll
            for (int m = 0; m < M; ++m) t[m] = dot2(p, xp[m][4 * wi + i], t[m]);
          }
        }
#pragma unroll
        for (int m = 0; m < M; ++m) acc[r][m] = fmaf(sc, fmaf(-off, xsum[m], t[m]), acc[r][m]);
      }
    }
  }

  // reduce across the wave
  float tot[RW][M];
#pragma unroll
  for (int r = 0; r < RW; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) tot[r][m] = wave_sum(acc[r][m]);

  float rs[RW];
#pragma unroll
  for (int r = 0; r < RW; ++r)
    rs[r] = (FMT == WQ_FMT_W8_PC) ? bf16_to_f32(scales[rown[r]]) : 1.f;

  if (split_k == 1) {
    if (lane == 0) {
#pragma unroll
      for (int r = 0; r < RW; ++r)
        if (n0 + r < N)
#pragma unroll
          for (int m = 0; m < M; ++m) y[(size_t)m * N + n0 + r] = f32_to_bf16(rs[r] * tot[r][m]);
    }
    return;
  }

  // split-K: publish this slice's partials, then the last slice to arrive reduces
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < RW; ++r)
      if (n0 + r < N)
#pragma unroll
        for (int m = 0; m < M; ++m) part[((size_t)s * M + m) * N + n0 + r] = tot[r][m];
  }
  __threadfence();
  uint32_t prev = 0;
  if (lane == 0) prev = atomicAdd(&counters[tile], 1u);
  prev = (uint32_t)__builtin_amdgcn_readfirstlane((int)prev);
  if (prev != (uint32_t)(split_k - 1)) return;
  __threadfence();
  if (lane < RW * M) {
    const int r = lane % RW, m = lane / RW;
    if (n0 + r < N) {
      float sum = 0.f;
      for (int t = 0; t < split_k; ++t) sum += part[((size_t)t * M + m) * N + n0 + r];
      const float sc = (FMT == WQ_FMT_W8_PC) ? bf16_to_f32(scales[n0 + r]) : 1.f;
      y[(size_t)m * N + n0 + r] = f32_to_bf16(sc * sum);
    }
  }
  if (lane == 0) __hip_atomic_store(&counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int FMT>
wq_status launch_fmt(const wq_weight* w, const uint16_t* x, int M, uint16_t* y, int split_k,
                     void* ws, hipStream_t st) {
  const int K = (int)w->K, N = (int)w->N;
  const int tiles = (N + RW - 1) / RW;
  dim3 grid((tiles + kWaves - 1) / kWaves, split_k);
  uint32_t* counters = (uint32_t*)ws;
  float* part = ws ? (float*)((char*)ws + kCounterBytes) : nullptr;
  const uint8_t* qw = (const uint8_t*)w->qweight;
  const uint16_t* sc = (const uint16_t*)w->scales;
  const uint8_t* zs = (const uint8_t*)w->zeros;
#define WQ_GEMV_CASE(MM)                                                                    \
  case MM:                                                                                  \
    gemv_kernel<FMT, MM><<<grid, 256, 0, st>>>(qw, sc, zs, x, y, counters, part, K, N, split_k); \
    break;
  switch (M) {
    WQ_GEMV_CASE(1)
    WQ_GEMV_CASE(2)
    WQ_GEMV_CASE(3)
    WQ_GEMV_CASE(4)
    WQ_GEMV_CASE(5)
    WQ_GEMV_CASE(6)
    WQ_GEMV_CASE(7)
    default:
      return fail(WQ_ERR_INVALID_ARG, "wq_gemv: M must be in 1..7");
  }
#undef WQ_GEMV_CASE
  WQ_HIP_CHECK(hipGetLastError());
  return WQ_OK;
}

}  // namespace

size_t gemv_workspace_bytes(int64_t N, int64_t M, int split_k) {
  if (split_k <= 1) return 0;
  return kCounterBytes + (size_t)split_k * (size_t)M * (size_t)N * sizeof(float);
}

int64_t gemv_max_rows() { return (int64_t)(kCounterBytes / sizeof(uint32_t)) * RW; }

wq_status launch_gemv(const wq_weight* w, const uint16_t* x, int M, uint16_t* y, int split_k,
                      void* ws, hipStream_t s) {
  switch (w->fmt) {
    case WQ_FMT_W8_PC: return launch_fmt<WQ_FMT_W8_PC>(w, x, M, y, split_k, ws, s);
    case WQ_FMT_W8_G128: return launch_fmt<WQ_FMT_W8_G128>(w, x, M, y, split_k, ws, s);
    case WQ_FMT_W4_G128: return launch_fmt<WQ_FMT_W4_G128>(w, x, M, y, split_k, ws, s);
  }
  return fail(WQ_ERR_UNSUPPORTED, "wq_gemv: unknown format");
}

}  // namespace wq
