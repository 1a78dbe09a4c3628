// Decode GEMV for 1 <= M <= 7 tokens: y[m][n] = sum_k x[m][k] * dequant(W)[n][k].
//
// Work decomposition (gfx950, wave64):
//   * A workgroup owns a tile of kGemvRowsPerWave (RW) consecutive output rows
//     and one split-K slice of K.  Its W waves (W = 1..16) interleave over the
//     slice in 1 KB steps: wave w reads chunks (i*W + w)*64 + lane, so at every
//     step the workgroup streams W contiguous kilobytes of each row with 128-bit
//     loads, and every lane reuses its x chunk for the RW rows.
//   * The loop is software-pipelined: the codes (and group metadata) and x of
//     the next step are in flight while the current step is multiplied.
//   * Codes become exact bf16 pairs in registers and meet bf16 x pairs in
//     v_dot2 (two multiply-adds, fp32 accumulate):
//       - int8: v_cvt_f32_i32 with a sign-extended byte select, then
//         v_cvt_pk_bf16_f32 (|q| <= 127 is exact in bf16);
//       - uint4 (nibbles interleaved by the gfx950 repack): (word >> 4i) &
//         0x000F000F | 0x43004300 is the bf16 pair (128 + q_2i, 128 + q_2i+1);
//         the offset is removed per 32-element chunk as (128 + z) * sum(x).
//   * Scales multiply fp32 partial sums (per row at the end for per-channel W8,
//     per chunk for group-128), so the codes stay exact.
//   * Each wave reduces its RW x M partials with DPP row operations and lane
//     reads; the W waves' partials meet in LDS and are summed in wave order.
//   * split_k > 1 splits K across workgroups: each slice writes fp32 partials
//     to the workspace and a second kernel sums them in slice order, so the
//     result is deterministic and no cross-workgroup fence is needed.
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

constexpr int RW = kGemvRowsPerWave;
constexpr int kMaxWaves = 16;

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
  p0 = pack_bf16x2((float)(int8_t)(d & 0xFFu), (float)(int8_t)((d >> 8) & 0xFFu));
  p1 = pack_bf16x2((float)(int8_t)((d >> 16) & 0xFFu), (float)(int8_t)(d >> 24));
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ float f16_to_f32(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }
__device__ __forceinline__ uint16_t f32_to_bf16(float v) {
  return __builtin_bit_cast(uint16_t, (__bf16)v);  // v_cvt_pk_bf16_f32: nearest even
}

#define WQ_DPP(v, ctrl) \
  __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), ctrl, 0xF, 0xF, false))

// Sum over the 64 lanes of a wave; the result is wave-uniform.
__device__ __forceinline__ float wave_sum(float v) {
  v += WQ_DPP(v, 0xB1);   // quad_perm [1,0,3,2]
  v += WQ_DPP(v, 0x4E);   // quad_perm [2,3,0,1]
  v += WQ_DPP(v, 0x141);  // row_half_mirror
  v += WQ_DPP(v, 0x140);  // row_mirror
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
  static constexpr int kPerChunk = 16;  // k values per 16-byte chunk of codes
  static constexpr int kChunksPerUnit = 1;
  static constexpr int kXWords = 8;     // uint32 (bf16 pairs) of x per chunk and token
};
template <>
struct Fmt<WQ_FMT_W8_G128> {
  static constexpr int kPerChunk = 16;
  static constexpr int kChunksPerUnit = 8;  // one 128-group
  static constexpr int kXWords = 8;
};
template <>
struct Fmt<WQ_FMT_W4_G128> {
  static constexpr int kPerChunk = 32;
  static constexpr int kChunksPerUnit = 4;
  static constexpr int kXWords = 16;
};

// Registers of one pipeline stage: codes of RW rows, x for M tokens, metadata.
template <int FMT, int M>
struct Stage {
  uint4 w[RW];
  uint32_t x[M][Fmt<FMT>::kXWords];
  uint16_t s[RW];
  uint8_t z[RW];
};

template <int FMT, int M>
__device__ __forceinline__ void load_stage(Stage<FMT, M>& st, const uint8_t* const* rowp,
                                           const int* rown, const uint16_t* __restrict__ x,
                                           const uint16_t* __restrict__ scales,
                                           const uint8_t* __restrict__ zeros, int K, int G, int Gh,
                                           int c) {
  using F = Fmt<FMT>;
#pragma unroll
  for (int r = 0; r < RW; ++r) st.w[r] = *reinterpret_cast<const uint4*>(rowp[r] + (size_t)c * 16);
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const uint4* xs = reinterpret_cast<const uint4*>(x + (size_t)m * K + (size_t)c * F::kPerChunk);
#pragma unroll
    for (int j = 0; j < F::kXWords / 4; ++j) {
      const uint4 a = xs[j];
      st.x[m][4 * j + 0] = a.x;
      st.x[m][4 * j + 1] = a.y;
      st.x[m][4 * j + 2] = a.z;
      st.x[m][4 * j + 3] = a.w;
    }
  }
  if constexpr (FMT == WQ_FMT_W8_G128) {
#pragma unroll
    for (int r = 0; r < RW; ++r) st.s[r] = scales[(size_t)rown[r] * G + (c >> 3)];
  } else if constexpr (FMT == WQ_FMT_W4_G128) {
    const int g = c >> 2;
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      st.s[r] = scales[(size_t)rown[r] * G + g];
      st.z[r] = zeros[(size_t)rown[r] * Gh + (g >> 1)];
    }
  }
}

template <int FMT, int M>
__device__ __forceinline__ void compute_stage(const Stage<FMT, M>& st, float (&acc)[RW][M], int c) {
  if constexpr (FMT != WQ_FMT_W4_G128) {
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      uint32_t wp[8];
      i8x4_to_bf16(st.w[r].x, wp[0], wp[1]);
      i8x4_to_bf16(st.w[r].y, wp[2], wp[3]);
      i8x4_to_bf16(st.w[r].z, wp[4], wp[5]);
      i8x4_to_bf16(st.w[r].w, wp[6], wp[7]);
      if constexpr (FMT == WQ_FMT_W8_PC) {
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[r][m] = dot2(wp[i], st.x[m][i], acc[r][m]);
      } else {
        const float sc = bf16_to_f32(st.s[r]);
#pragma unroll
        for (int m = 0; m < M; ++m) {
          float t = 0.f;
#pragma unroll
          for (int i = 0; i < 8; ++i) t = dot2(wp[i], st.x[m][i], t);
          acc[r][m] = fmaf(sc, t, acc[r][m]);
        }
      }
    }
  } else {
    float xsum[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float t = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) t = dot2(st.x[m][i], 0x3F803F80u, t);  // x . (1, 1)
      xsum[m] = t;
    }
    const int g = c >> 2;
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      const float sc = f16_to_f32(st.s[r]);
      const float off = 128.f + (float)((st.z[r] >> ((g & 1) * 4)) & 0xFu);
      const uint32_t words[4] = {st.w[r].x, st.w[r].y, st.w[r].z, st.w[r].w};
      float t[M];
#pragma unroll
      for (int m = 0; m < M; ++m) t[m] = 0.f;
#pragma unroll
      for (int wi = 0; wi < 4; ++wi) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t p = ((words[wi] >> (4 * i)) & 0x000F000Fu) | 0x43004300u;
#pragma unroll
          for (int m = 0; m < M; ++m) t[m] = dot2(p, st.x[m][4 * wi + i], t[m]);
        }
      }
#pragma unroll
      for (int m = 0; m < M; ++m) acc[r][m] = fmaf(sc, fmaf(-off, xsum[m], t[m]), acc[r][m]);
    }
  }
}

// grid = (row tiles, split_k); block = 64 * W threads, W <= MAXW (the register
// budget per thread shrinks as the workgroup grows: 512 VGPRs per SIMD lane are
// shared by the W/4 waves a SIMD hosts).
template <int FMT, int M, int MAXW>
__global__ __launch_bounds__(64 * MAXW) void gemv_kernel(const uint8_t* __restrict__ qw,
                                                      const uint16_t* __restrict__ scales,
                                                      const uint8_t* __restrict__ zeros,
                                                      const uint16_t* __restrict__ x,
                                                      uint16_t* __restrict__ y,
                                                      float* __restrict__ part, int K, int N) {
  using F = Fmt<FMT>;
  __shared__ float red[MAXW][RW * M];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int W = blockDim.x >> 6;
  const int n0 = blockIdx.x * RW;
  const int s = blockIdx.y, S = gridDim.y;

  const int chunks_row = K / F::kPerChunk;
  const int units = chunks_row / F::kChunksPerUnit;
  const int c0 = (int)(((int64_t)s * units) / S) * F::kChunksPerUnit;
  const int c1 = (int)(((int64_t)(s + 1) * units) / S) * F::kChunksPerUnit;
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

  // Two register stages in ping-pong: the loads of one are in flight while the
  // other is multiplied.  The loop is counted so that every prefetched stage is
  // consumed (the compiler then keeps the prefetch ahead of the math and the wait
  // counters only wait for the older stage).
  const int step = 64 * W;
  const int cfirst = c0 + wave * 64 + lane;
  const int n = cfirst < c1 ? (c1 - cfirst + step - 1) / step : 0;  // chunks of this lane
  if (n > 0) {
    Stage<FMT, M> A, B;
    int c = cfirst;
    load_stage<FMT, M>(A, rowp, rown, x, scales, zeros, K, G, Gh, c);
    int left = n;  // stages not yet multiplied, the first of them in A
    while (left >= 3) {
      load_stage<FMT, M>(B, rowp, rown, x, scales, zeros, K, G, Gh, c + step);
      compute_stage<FMT, M>(A, acc, c);
      load_stage<FMT, M>(A, rowp, rown, x, scales, zeros, K, G, Gh, c + 2 * step);
      compute_stage<FMT, M>(B, acc, c + step);
      c += 2 * step;
      left -= 2;
    }
    if (left == 2) {
      load_stage<FMT, M>(B, rowp, rown, x, scales, zeros, K, G, Gh, c + step);
      compute_stage<FMT, M>(A, acc, c);
      compute_stage<FMT, M>(B, acc, c + step);
    } else {
      compute_stage<FMT, M>(A, acc, c);
    }
  }

  float tot[RW][M];
#pragma unroll
  for (int r = 0; r < RW; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) tot[r][m] = wave_sum(acc[r][m]);

  const int t = threadIdx.x;
  float v = 0.f;
  if (W == 1) {
    // lane j < RW*M takes (r, m) = (j % RW, j / RW); values are wave-uniform
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
      for (int m = 0; m < M; ++m)
        if (t == m * RW + r) v = tot[r][m];
  } else {
    if (lane == 0) {
#pragma unroll
      for (int r = 0; r < RW; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) red[wave][m * RW + r] = tot[r][m];
    }
    __syncthreads();
    if (t < RW * M)
      for (int w = 0; w < W; ++w) v += red[w][t];
  }
  if (t < RW * M) {
    const int r = t % RW, m = t / RW, n = n0 + r;
    if (n < N) {
      if (S == 1) {
        const float sc = (FMT == WQ_FMT_W8_PC) ? bf16_to_f32(scales[n]) : 1.f;
        y[(size_t)m * N + n] = f32_to_bf16(sc * v);
      } else {
        part[((size_t)s * M + m) * N + n] = v;
      }
    }
  }
}

// y[m][n] = bf16(scale[n] * sum_s part[s][m][n]), slices summed in order.
template <int FMT>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part,
                                                              const uint16_t* __restrict__ scales,
                                                              uint16_t* __restrict__ y, int M,
                                                              int N, int S) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t MN = (int64_t)M * N;
  if (i >= MN) return;
  float v = 0.f;
  for (int s = 0; s < S; ++s) v += part[(int64_t)s * MN + i];
  const int n = (int)(i % N);
  const float sc = (FMT == WQ_FMT_W8_PC) ? bf16_to_f32(scales[n]) : 1.f;
  y[i] = f32_to_bf16(sc * v);
}

// Largest waves per workgroup whose register budget (512 / (W/4) VGPRs per lane)
// holds this format and M without spilling.
constexpr int max_waves(int fmt, int M) {
  return fmt == WQ_FMT_W8_PC ? (M <= 4 ? 16 : 8)
         : fmt == WQ_FMT_W8_G128 ? (M <= 3 ? 16 : 8)
                                 : (M <= 1 ? 16 : M <= 5 ? 8 : 4);
}

template <int FMT>
wq_status launch_fmt(const wq_weight* w, const uint16_t* x, int M, uint16_t* y, int split_k,
                     int waves, void* ws, hipStream_t st) {
  const int K = (int)w->K, N = (int)w->N;
  const int tiles = (N + RW - 1) / RW;
  dim3 grid(tiles, split_k);
  dim3 block(64 * waves);
  float* part = (float*)ws;
  const uint8_t* qw = (const uint8_t*)w->qweight;
  const uint16_t* sc = (const uint16_t*)w->scales;
  const uint8_t* zs = (const uint8_t*)w->zeros;
#define WQ_GEMV_CASE(MM)                                                                     \
  case MM:                                                                                   \
    if (waves <= 4)                                                                          \
      gemv_kernel<FMT, MM, 4><<<grid, block, 0, st>>>(qw, sc, zs, x, y, part, K, N);        \
    else if constexpr (max_waves(FMT, MM) >= 8) {                                            \
      if (waves <= 8)                                                                        \
        gemv_kernel<FMT, MM, 8><<<grid, block, 0, st>>>(qw, sc, zs, x, y, part, K, N);      \
      else if constexpr (max_waves(FMT, MM) >= 16)                                           \
        gemv_kernel<FMT, MM, 16><<<grid, block, 0, st>>>(qw, sc, zs, x, y, part, K, N);     \
    }                                                                                        \
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
  if (split_k > 1) {
    const int64_t MN = (int64_t)M * N;
    splitk_reduce_kernel<FMT><<<(unsigned)((MN + 255) / 256), 256, 0, st>>>(part, sc, y, M, N, split_k);
    WQ_HIP_CHECK(hipGetLastError());
  }
  return WQ_OK;
}

}  // namespace

size_t gemv_workspace_bytes(int64_t N, int64_t M, int split_k) {
  if (split_k <= 1) return 0;
  return (size_t)split_k * (size_t)M * (size_t)N * sizeof(float);
}

int gemv_max_waves(int fmt, int M) { return max_waves(fmt, M); }

int gemv_default_waves(int64_t K, int64_t N, int fmt, int M, int split_k) {
  // aim at about 8192 resident waves (32 per CU) with at least two 1-KB steps
  // of each row per wave
  const int64_t tiles = (N + RW - 1) / RW;
  const int64_t per_chunk = fmt == WQ_FMT_W4_G128 ? 32 : 16;
  const int64_t slice_chunks = (K / per_chunk) / split_k;
  const int cap = gemv_max_waves(fmt, M);
  int w = 1;
  while (w < cap && tiles * split_k * (w * 2) <= 8192 && slice_chunks >= (int64_t)(w * 2) * 128) w *= 2;
  return w;
}

wq_status launch_gemv(const wq_weight* w, const uint16_t* x, int M, uint16_t* y, int split_k,
                      int waves, void* ws, hipStream_t s) {
  if (waves < 1 || waves > kMaxWaves || (waves & (waves - 1)))
    return fail(WQ_ERR_INVALID_ARG, "wq_gemv: waves per workgroup must be 1, 2, 4, 8 or 16");
  if (waves > gemv_max_waves(w->fmt, M))
    return fail(WQ_ERR_UNSUPPORTED, "wq_gemv: at this M a workgroup holds at most " +
                                        std::to_string(gemv_max_waves(w->fmt, M)) + " waves");
  switch (w->fmt) {
    case WQ_FMT_W8_PC: return launch_fmt<WQ_FMT_W8_PC>(w, x, M, y, split_k, waves, ws, s);
    case WQ_FMT_W8_G128: return launch_fmt<WQ_FMT_W8_G128>(w, x, M, y, split_k, waves, ws, s);
    case WQ_FMT_W4_G128: return launch_fmt<WQ_FMT_W4_G128>(w, x, M, y, split_k, waves, ws, s);
  }
  return fail(WQ_ERR_UNSUPPORTED, "wq_gemv: unknown format");
}

}  // namespace wq
