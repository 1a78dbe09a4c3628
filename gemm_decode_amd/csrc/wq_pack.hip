// Quantize-and-pack kernels (canonical layout) and the canonical <-> gfx950 repack.
//
// The formats are those of the tileInfer README (feature table, "INT8 Weight-Only
// Quantization": int8 codes with one scale per output channel) and of "Marlin
// register and launch scheduling benchmark" ("Validation and limits": INT8/INT4
// with per-channel or group-128 scales).  The pages print no quantization
// arithmetic; the recipe implemented here is the one stated at wq_pack in wq.h:
// IEEE fp32, round to nearest even, correctly rounded division by the stored
// (rounded) scale.
#include "wq_internal.h"

namespace wq {
namespace {

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float v) {
  uint32_t u = __float_as_uint(v);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ uint16_t f32_to_f16_rne(float v) {
  _Float16 h = (_Float16)v;  // v_cvt_f16_f32, round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float f16_to_f32(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

// Max over the `width` lanes of a sub-wave (width a power of two <= 64).
template <int WIDTH>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int o = WIDTH / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WIDTH));
  return v;
}
template <int WIDTH>
__device__ __forceinline__ float group_min(float v) {
#pragma unroll
  for (int o = WIDTH / 2; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o, WIDTH));
  return v;
}

// Four consecutive weights as fp32: fp32 input as is, bf16 input widened (exact).
__device__ __forceinline__ float4 load_w4(const float* w, size_t off) {
  return *reinterpret_cast<const float4*>(w + off);
}
__device__ __forceinline__ float4 load_w4(const uint16_t* w, size_t off) {
  const uint2 v = *reinterpret_cast<const uint2*>(w + off);
  return make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xFFFF0000u), __uint_as_float(v.y << 16),
                     __uint_as_float(v.y & 0xFFFF0000u));
}

__device__ __forceinline__ uint32_t w8_codes4(float4 w, float s) {
  // q = clamp(rint(w / s), -127, 127); s != 0 here.
  float c[4] = {w.x, w.y, w.z, w.w};
  uint32_t out = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float q = fminf(fmaxf(rintf(c[j] / s), -127.f), 127.f);
    out |= ((uint32_t)(int32_t)q & 0xFFu) << (8 * j);
  }
  return out;
}

// W8, one scale per output channel: one 256-thread block per row.
template <typename T>
__global__ __launch_bounds__(256) void pack_w8_pc_kernel(const T* __restrict__ w,
                                                           int8_t* __restrict__ q,
                                                           uint16_t* __restrict__ scales, int K) {
  const int n = blockIdx.x;
  const size_t row = (size_t)n * K;
  uint32_t* qrow = reinterpret_cast<uint32_t*>(q + (size_t)n * K);
  const int words = K / 4;
  float a = 0.f;
  for (int i = threadIdx.x; i < words; i += 256) {
    float4 v = load_w4(w, row + 4 * (size_t)i);
    a = fmaxf(a, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
  }
  a = group_max<64>(a);
  __shared__ float red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = a;
  __syncthreads();
  a = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const uint16_t sb = f32_to_bf16_rne(a / 127.f);
  const float s = bf16_to_f32(sb);
  if (threadIdx.x == 0) scales[n] = sb;
  for (int i = threadIdx.x; i < words; i += 256) qrow[i] = (s == 0.f) ? 0u : w8_codes4(load_w4(w, row + 4 * (size_t)i), s);
}

// W8 with groups of GS (32, 64, 128) k: 256 threads = 256 / (GS / 4) groups of GS / 4
// lanes, each lane 4 consecutive k.
template <typename T, int GS>
__global__ __launch_bounds__(256) void pack_w8_g_kernel(const T* __restrict__ w,
                                                          int8_t* __restrict__ q,
                                                          uint16_t* __restrict__ scales,
                                                          int K, int N) {
  constexpr int L = GS / 4;  // lanes per group
  const int G = K / GS;
  const int64_t gid = (int64_t)blockIdx.x * (256 / L) + (threadIdx.x / L);
  const int lane = threadIdx.x % L;
  const bool valid = gid < (int64_t)N * G;
  const int64_t gg = valid ? gid : 0;
  const int64_t n = gg / G, g = gg % G;
  const size_t off = (size_t)n * K + (size_t)g * GS + 4 * lane;
  float4 v = load_w4(w, off);
  float a = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
  a = group_max<L>(a);
  const uint16_t sb = f32_to_bf16_rne(a / 127.f);
  const float s = bf16_to_f32(sb);
  if (!valid) return;
  if (lane == 0) scales[n * G + g] = sb;
  *reinterpret_cast<uint32_t*>(q + off) = (s == 0.f) ? 0u : w8_codes4(v, s);
}

// W4 asymmetric with groups of GS (32, 64, 128) k, canonical layout: a block of 2 GS
// threads handles 8 rows x 1 group, GS / 4 lanes per row, 4 consecutive k per lane; the
// 8 zero-points form one word.
template <typename T, int GS>
__global__ __launch_bounds__(2 * GS) void pack_w4_g_kernel(const T* __restrict__ w,
                                                             uint32_t* __restrict__ qw,
                                                             uint16_t* __restrict__ scales,
                                                             uint32_t* __restrict__ zeros, int K,
                                                             int N) {
  constexpr int L = GS / 4;  // lanes per row
  const int G = K / GS;
  const int c8 = blockIdx.x;  // rows 8*c8 .. 8*c8+7
  const int g = blockIdx.y;
  const int r = threadIdx.x / L, lane = threadIdx.x % L;
  const int n = 8 * c8 + r;
  const size_t off = (size_t)n * K + (size_t)g * GS + 4 * lane;
  float4 v = load_w4(w, off);
  float hi = group_max<L>(fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w)));
  float lo = group_min<L>(fminf(fminf(v.x, v.y), fminf(v.z, v.w)));
  const uint16_t sh = f32_to_f16_rne((hi - lo) / 15.f);
  const float s = f16_to_f32(sh);
  uint32_t z = 0, nib = 0;
  if (s != 0.f) {
    z = (uint32_t)fminf(fmaxf(rintf(-lo / s), 0.f), 15.f);
    float c[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float qq = fminf(fmaxf(rintf(c[j] / s) + (float)z, 0.f), 15.f);
      nib |= ((uint32_t)qq) << (4 * j);
    }
  }
  // lanes 2i and 2i+1 hold k = 8i..8i+3 and 8i+4..8i+7 of the same word
  const uint32_t partner = (uint32_t)__shfl_xor((int)nib, 1, L);
  if ((lane & 1) == 0) qw[(size_t)n * (K / 8) + (size_t)g * (GS / 8) + (lane >> 1)] = nib | (partner << 16);
  __shared__ uint32_t zs[8];
  if (lane == 0) {
    scales[(size_t)n * G + g] = sh;
    zs[r] = z;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) word |= zs[j] << (4 * j);
    zeros[(size_t)g * (N / 8) + c8] = word;
  }
}

// W4 asymmetric per output channel, canonical layout: a block handles 8 rows, 32 lanes
// per row, each lane 4 consecutive k of every 128 (one pass for the row's min and max,
// a second for the codes); the 8 zero-points form one word.
template <typename T>
__global__ __launch_bounds__(256) void pack_w4_pc_kernel(const T* __restrict__ w, uint32_t* __restrict__ qw,
                                                           uint16_t* __restrict__ scales,
                                                           uint32_t* __restrict__ zeros, int K) {
  const int G = K / kGroup;
  const int c8 = blockIdx.x;  // rows 8*c8 .. 8*c8+7
  const int r = threadIdx.x >> 5, lane = threadIdx.x & 31;
  const int n = 8 * c8 + r;
  const size_t row = (size_t)n * K + 4 * lane;
  float hi = -INFINITY, lo = INFINITY;
  for (int g = 0; g < G; ++g) {
    const float4 v = load_w4(w, row + (size_t)g * kGroup);
    hi = fmaxf(hi, fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w)));
    lo = fminf(lo, fminf(fminf(v.x, v.y), fminf(v.z, v.w)));
  }
  hi = group_max<32>(hi);
  lo = group_min<32>(lo);
  const uint16_t sh = f32_to_f16_rne((hi - lo) / 15.f);
  const float s = f16_to_f32(sh);
  const uint32_t z = s != 0.f ? (uint32_t)fminf(fmaxf(rintf(-lo / s), 0.f), 15.f) : 0u;
  for (int g = 0; g < G; ++g) {
    uint32_t nib = 0;
    if (s != 0.f) {
      const float4 v = load_w4(w, row + (size_t)g * kGroup);
      const float c[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float qq = fminf(fmaxf(rintf(c[j] / s) + (float)z, 0.f), 15.f);
        nib |= ((uint32_t)qq) << (4 * j);
      }
    }
    // lanes 2i and 2i+1 hold k = 8i..8i+3 and 8i+4..8i+7 of the same word
    const uint32_t partner = (uint32_t)__shfl_xor((int)nib, 1, 32);
    if ((lane & 1) == 0) qw[(size_t)n * (K / 8) + (size_t)g * 16 + (lane >> 1)] = nib | (partner << 16);
  }
  __shared__ uint32_t zs[8];
  if (lane == 0) {
    scales[n] = sh;
    zs[r] = z;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) word |= zs[j] << (4 * j);
    zeros[c8] = word;
  }
}

// Nibble position p of a gfx950 W4 word holds canonical nibble kPerm[p].
__device__ __forceinline__ uint32_t nibbles_to_gfx950(uint32_t c) {
  uint32_t o = 0;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int src = (p < 4) ? 2 * p : 2 * (p - 4) + 1;
    o |= ((c >> (4 * src)) & 0xFu) << (4 * p);
  }
  return o;
}
__device__ __forceinline__ uint32_t nibbles_from_gfx950(uint32_t o) {
  uint32_t c = 0;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int dst = (p < 4) ? 2 * p : 2 * (p - 4) + 1;
    c |= ((o >> (4 * p)) & 0xFu) << (4 * dst);
  }
  return c;
}

// Codes, one 16-byte chunk per thread: canonical row-major [N][row_bytes] <->
// gfx950 tiled order (tiled_offset); int8 codes get their sign bit flipped
// (u = q + 128), uint4 words get their nibbles interleaved.
template <bool W4>
__global__ void codes_repack_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                    int64_t N, int64_t row_bytes, int to_gfx950) {
  const int64_t chunks_row = row_bytes / 16;
  const size_t total = (size_t)N * chunks_row;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (size_t)gridDim.x * blockDim.x) {
    const int64_t n = (int64_t)(i / chunks_row), b = (int64_t)(i % chunks_row) * 16;
    const size_t lin = (size_t)n * row_bytes + b, til = tiled_offset(n, b, N, row_bytes);
    uint4 v = *reinterpret_cast<const uint4*>(src + (to_gfx950 ? lin : til));
    if (W4) {
      if (to_gfx950) {
        v.x = nibbles_to_gfx950(v.x); v.y = nibbles_to_gfx950(v.y);
        v.z = nibbles_to_gfx950(v.z); v.w = nibbles_to_gfx950(v.w);
      } else {
        v.x = nibbles_from_gfx950(v.x); v.y = nibbles_from_gfx950(v.y);
        v.z = nibbles_from_gfx950(v.z); v.w = nibbles_from_gfx950(v.w);
      }
    } else {
      v.x ^= 0x80808080u; v.y ^= 0x80808080u; v.z ^= 0x80808080u; v.w ^= 0x80808080u;
    }
    *reinterpret_cast<uint4*>(dst + (to_gfx950 ? til : lin)) = v;
  }
}

// Group scales: canonical [N][Gc]  <->  gfx950 tiles [N16][G][16] (16 rows of one
// group side by side; rows past N hold 0).  Gc = G, or 1 for per-channel W4, whose one
// scale per row fills every group of the tiles (and is read back from group 0).
__global__ void scales_tile_kernel(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst,
                                   int N, int G, int Gc, int to_tiled) {
  const size_t total = to_tiled ? (size_t)row_tiles(N) * G * kGemvTileRows : (size_t)N * Gc;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (size_t)gridDim.x * blockDim.x) {
    if (to_tiled) {
      const size_t t = i / ((size_t)G * kGemvTileRows), rem = i % ((size_t)G * kGemvTileRows);
      const int g = (int)(rem / kGemvTileRows), j = (int)(rem % kGemvTileRows);
      const size_t n = t * kGemvTileRows + j;
      dst[i] = n < (size_t)N ? src[n * Gc + (Gc == 1 ? 0 : g)] : (uint16_t)0;
    } else {
      const size_t n = i / Gc, g = i % Gc;
      dst[i] = src[((n / kGemvTileRows) * G + g) * kGemvTileRows + n % kGemvTileRows];
    }
  }
}

// canonical zeros uint32 [Gc][N/8]  ->  gfx950 zeros uint8 [N16][G][8], byte (t,g,h)
// holding z[16t+2h][g] (bits 0..3) and z[16t+2h+1][g] (bits 4..7); Gc = G, or 1 for
// per-channel W4 (its one zero-point per row in every group)
__global__ void w4_zeros_to_gfx950_kernel(const uint32_t* __restrict__ zc, uint8_t* __restrict__ zt,
                                          int G, int Gc, int N) {
  const size_t total = (size_t)row_tiles(N) * G * (kGemvTileRows / 2);
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (size_t)gridDim.x * blockDim.x) {
    const size_t t = i / ((size_t)G * 8), rem = i % ((size_t)G * 8);
    const int g = (int)(rem / 8), h = (int)(rem % 8);
    uint32_t b = 0;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const size_t n = t * kGemvTileRows + 2 * h + e;
      if (n < (size_t)N) b |= ((zc[(size_t)(Gc == 1 ? 0 : g) * (N / 8) + n / 8] >> (4 * (n % 8))) & 0xFu) << (4 * e);
    }
    zt[i] = (uint8_t)b;
  }
}

// gfx950 zeros uint8 [N16][G][8]  ->  canonical zeros uint32 [Gc][N/8] (groups 0 .. Gc - 1)
__global__ void w4_zeros_from_gfx950_kernel(const uint8_t* __restrict__ zt, uint32_t* __restrict__ zc,
                                            int G, int Gc, int N) {
  const size_t total = (size_t)Gc * (N / 8);
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (size_t)gridDim.x * blockDim.x) {
    const int g = (int)(i / (N / 8)), c = (int)(i % (N / 8));
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const size_t n = (size_t)8 * c + j;
      const uint8_t b = zt[((n / kGemvTileRows) * G + g) * 8 + (n % kGemvTileRows) / 2];
      word |= (uint32_t)((b >> (4 * (n & 1))) & 0xF) << (4 * j);
    }
    zc[i] = word;
  }
}

unsigned grid_for(size_t n, unsigned block) {
  size_t b = (n + block - 1) / block;
  if (b > 65535u * 16u) b = 65535u * 16u;
  return (unsigned)(b ? b : 1);
}

}  // namespace

template <typename T>
static wq_status launch_pack_t(const T* w, const wq_weight* out, hipStream_t s) {
  const int K = (int)out->K, N = (int)out->N;
  switch (out->fmt) {
    case WQ_FMT_W8_PC:
      pack_w8_pc_kernel<T><<<N, 256, 0, s>>>(w, (int8_t*)out->qweight, (uint16_t*)out->scales, K);
      break;
    case WQ_FMT_W8_G32:
    case WQ_FMT_W8_G64:
    case WQ_FMT_W8_G128: {
      const int gs = meta_group(out->fmt);
      const int64_t groups = (int64_t)N * (K / gs), per_block = 256 / (gs / 4);
      const unsigned blocks = (unsigned)((groups + per_block - 1) / per_block);
      int8_t* q = (int8_t*)out->qweight;
      uint16_t* sc = (uint16_t*)out->scales;
      if (gs == 32) pack_w8_g_kernel<T, 32><<<blocks, 256, 0, s>>>(w, q, sc, K, N);
      else if (gs == 64) pack_w8_g_kernel<T, 64><<<blocks, 256, 0, s>>>(w, q, sc, K, N);
      else pack_w8_g_kernel<T, 128><<<blocks, 256, 0, s>>>(w, q, sc, K, N);
      break;
    }
    case WQ_FMT_W4_G32:
    case WQ_FMT_W4_G64:
    case WQ_FMT_W4_G128: {
      const int gs = meta_group(out->fmt);
      const dim3 grid(N / 8, K / gs);
      uint32_t* q = (uint32_t*)out->qweight;
      uint16_t* sc = (uint16_t*)out->scales;
      uint32_t* z = (uint32_t*)out->zeros;
      if (gs == 32) pack_w4_g_kernel<T, 32><<<grid, 64, 0, s>>>(w, q, sc, z, K, N);
      else if (gs == 64) pack_w4_g_kernel<T, 64><<<grid, 128, 0, s>>>(w, q, sc, z, K, N);
      else pack_w4_g_kernel<T, 128><<<grid, 256, 0, s>>>(w, q, sc, z, K, N);
      break;
    }
    case WQ_FMT_W4_PC:
      pack_w4_pc_kernel<T><<<N / 8, 256, 0, s>>>(w, (uint32_t*)out->qweight, (uint16_t*)out->scales,
                                                (uint32_t*)out->zeros, K);
      break;
    default:
      return fail(WQ_ERR_UNSUPPORTED, "wq_pack: unknown format");
  }
  WQ_HIP_CHECK(hipGetLastError());
  return WQ_OK;
}

wq_status launch_pack(const float* w, const wq_weight* out, hipStream_t s) { return launch_pack_t(w, out, s); }
wq_status launch_pack_bf16(const uint16_t* w, const wq_weight* out, hipStream_t s) {
  return launch_pack_t(w, out, s);
}

wq_status launch_repack(const wq_weight* src, const wq_weight* dst, bool to_gfx950, hipStream_t s) {
  size_t qb = 0, sb = 0, zb = 0;
  wq_status st = wq_packed_sizes(src->fmt, WQ_LAYOUT_CANONICAL, src->K, src->N, &qb, &sb, &zb);
  if (st != WQ_OK) return st;
  const int gs = meta_group(src->fmt);  // 0 for per-channel W8 (its scales are copied)
  const int G = gs ? (int)(src->K / gs) : 0, N = (int)src->N;
  const int Gc = src->fmt == WQ_FMT_W4_PC ? 1 : G;  // canonical groups per row
  const int64_t row_bytes = (int64_t)(qb / (size_t)N);
  const size_t chunks = qb / 16;
  // codes
  if (is_w4(src->fmt)) {
    codes_repack_kernel<true><<<grid_for(chunks, 256), 256, 0, s>>>(
        (const uint8_t*)src->qweight, (uint8_t*)dst->qweight, N, row_bytes, to_gfx950);
  } else {
    codes_repack_kernel<false><<<grid_for(chunks, 256), 256, 0, s>>>(
        (const uint8_t*)src->qweight, (uint8_t*)dst->qweight, N, row_bytes, to_gfx950);
  }
  WQ_HIP_CHECK(hipGetLastError());
  // scales
  if (src->fmt == WQ_FMT_W8_PC) {
    WQ_HIP_CHECK(hipMemcpyAsync(dst->scales, src->scales, sb, hipMemcpyDeviceToDevice, s));
  } else {
    const size_t n = to_gfx950 ? (size_t)row_tiles(N) * G * kGemvTileRows : (size_t)N * Gc;
    scales_tile_kernel<<<grid_for(n, 256), 256, 0, s>>>((const uint16_t*)src->scales,
                                                        (uint16_t*)dst->scales, N, G, Gc, to_gfx950);
    WQ_HIP_CHECK(hipGetLastError());
  }
  // zero-points
  if (is_w4(src->fmt)) {
    if (to_gfx950) {
      w4_zeros_to_gfx950_kernel<<<grid_for((size_t)row_tiles(N) * G * 8, 256), 256, 0, s>>>(
          (const uint32_t*)src->zeros, (uint8_t*)dst->zeros, G, Gc, N);
    } else {
      w4_zeros_from_gfx950_kernel<<<grid_for((size_t)Gc * (N / 8), 256), 256, 0, s>>>(
          (const uint8_t*)src->zeros, (uint32_t*)dst->zeros, G, Gc, N);
    }
    WQ_HIP_CHECK(hipGetLastError());
  }
  return WQ_OK;
}

}  // namespace wq
