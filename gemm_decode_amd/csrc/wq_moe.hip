// Grouped (mixture-of-experts) weight-only linear, and its SiLU-gated epilogue.
//
// E experts of one format and shape (K, N) are stored one after another in the gfx950
// layout; the token rows of x are grouped by expert, expert e owning rows
// offsets[e] .. offsets[e + 1] - 1 (offsets on the device, so a routing computed there
// needs no copy to the host).  One launch covers every expert:
//
//   grid (tile pairs, E), 8 waves: a workgroup takes expert blockIdx.y and two 16-row
//   weight tiles -- tiles 2 b and 2 b + 1, or, for the gated epilogue, gate tile b and
//   the matching up tile b + I / 16 (N = 2 I: gate rows, then up rows) -- and walks the
//   expert's rows in blocks of 16 tokens (the A rows of v_mfma_f32_16x16x32), its
//   waves interleaving over 128-k units; an expert without rows leaves at once.
//
// The arithmetic is the matrix-core decode GEMV's: codes become exact fp16 values (int8
// by v_perm_b32 under the fp16 exponent byte and one packed fp16 add of -1152; uint4
// pairs under the fp16 1024.0 / 64.0 patterns and one packed add of -(1024 + z) /
// -(64 + z)) against x converted to fp16; a unit whose x fp16 cannot hold exactly takes
// exact bf16 codes against bf16 x.  Group scales multiply each unit's fp32 partial,
// per-channel scales the finished sum.  The four waves' sums meet in LDS; the epilogue
// writes y = bf16(sum), or, gated, h = bf16(silu(g) * u) from the fp32 gate and up sums
// (silu(v) = v / (1 + exp(-v))), so the gate and up outputs never leave the kernel.
//
// Prior art: the Marlin register and launch scheduling benchmark page validates a shared
// MoE kernel beside its dense one ("Validation and limits"); the SGLang quantization
// stack review argues for one shared WnA16 kernel across formats (Figure 4 comments);
// the tileInfer README fuses the SiLU gate ("Key Optimizations").  Nothing here follows
// their code.
#include "wq_internal.h"

namespace wq {
namespace {

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kMoeWaves = 8;
constexpr int kMoeTokens = 16;  // tokens per block (A rows of one matrix instruction)

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ float f16_to_f32(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }
__device__ __forceinline__ uint16_t f32_to_bf16(float v) { return __builtin_bit_cast(uint16_t, (__bf16)v); }
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v;
  v.x = (__bf16)lo;
  v.y = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}
// bf16 pair -> fp16 pair (exact for the values F16Exact accepts)
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(__uint_as_float(b << 16),
                                                                 __uint_as_float(b & 0xFFFF0000u)));
}
__device__ __forceinline__ uint32_t add_f16x2(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, a) + __builtin_bit_cast(f16x2_t, b));
}
constexpr uint32_t kF16Minus1152 = 0xE480E480u;  // fp16 pair (-1152, -1152)

// every bf16 value added is 0 or lies in [2^-17, 65280] (fp16 holds it exactly)
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

__device__ __forceinline__ f32x4_t mma_f16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                0, 0, 0);
}
__device__ __forceinline__ f32x4_t mma_bf16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                 c, 0, 0, 0);
}
// exact bf16 pairs of four signed codes stored as u = q + 128
__device__ __forceinline__ void i8_word_to_bf16(uint32_t d, uint32_t& lo, uint32_t& hi) {
  d ^= 0x80808080u;
  lo = pack_bf16x2((float)(int8_t)(d & 0xFFu), (float)(int8_t)((d >> 8) & 0xFFu));
  hi = pack_bf16x2((float)(int8_t)((d >> 16) & 0xFFu), (float)(int8_t)(d >> 24));
}

// grid (pairs, E); block 64 W, W <= kMoeWaves, with W * 2 KiB of dynamic LDS for the
// waves' sums.  K % 128 == 0, N % 16 == 0 (and, gated, (N / 2) % 16 == 0), checked on the
// host.  Offsets are clamped into [0, T] before use.
template <int FMT, bool GATED, int MB>
__global__ __launch_bounds__(64 * kMoeWaves) void moe_kernel(const uint8_t* __restrict__ qw0,
                                                            const uint16_t* __restrict__ sc0,
                                                            const uint8_t* __restrict__ zs0, size_t qw_stride,
                                                            size_t sc_stride, size_t zs_stride,
                                                            const uint16_t* __restrict__ x,
                                                            const int32_t* __restrict__ offsets,
                                                            uint16_t* __restrict__ y, int T, int K, int N) {
  constexpr bool kW4 = FMT == WQ_FMT_W4_G128, kGrouped = FMT != WQ_FMT_W8_PC;
  constexpr int kUnitBytes = kW4 ? 64 : 128;  // code bytes per row and 128-k unit
  constexpr int kUnitsPerSlice = kSliceBytes / kUnitBytes;
  constexpr int CL = kW4 ? 1 : 2;             // 16-byte code loads per lane, tile and unit
  extern __shared__ float red[];  // [W][2][kMoeTokens][16]

  const int e = blockIdx.y;
  const int t0 = min(max(offsets[e], 0), T);
  const int t1 = min(max(offsets[e + 1], t0), T);
  if (t1 <= t0) return;  // the whole workgroup leaves together

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, W = blockDim.x >> 6;
  const int wu = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t ln = lane & 15, lk = lane >> 4;
  const int T16 = N / 16, G = K / kGroup, U = K / kGroup;
  const uint32_t row_bytes = kW4 ? (uint32_t)K / 2 : (uint32_t)K;
  // the two tiles: gate and up (gated), else two neighbours (the second may not exist)
  int tt[2];
  tt[0] = GATED ? (int)blockIdx.x : 2 * (int)blockIdx.x;
  tt[1] = GATED ? (int)blockIdx.x + T16 / 2 : min(2 * (int)blockIdx.x + 1, T16 - 1);
  const bool second = GATED || 2 * (int)blockIdx.x + 1 < T16;

  const uint8_t* qw = qw0 + (size_t)e * qw_stride;
  const uint16_t* sc = reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(sc0) + (size_t)e * sc_stride);
  const uint8_t* zs = kW4 ? zs0 + (size_t)e * zs_stride : nullptr;
  const uint8_t* tbase[2];
  const uint16_t* sbase[2];
  const uint8_t* zbase[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    tbase[t] = qw + (size_t)tt[t] * 16 * row_bytes;
    sbase[t] = kGrouped ? sc + (size_t)tt[t] * G * 16 : sc;
    zbase[t] = kW4 ? zs + (size_t)tt[t] * G * 8 : nullptr;
  }
  const uint32_t zshift = 4 * (ln & 1);
  uint32_t m_lo = 0x000F000Fu, m_hi = 0x00F000F0u, mag_a = 0x64006400u, mag_h = 0x54005400u;
  if constexpr (kW4) asm volatile("" : "+v"(m_lo), "+v"(m_hi), "+v"(mag_a), "+v"(mag_h));

  // One unit's operands: both tiles' codes, their group scales and zero bytes.  The
  // codes become the B operands once per unit and feed the MFMAs of every token block.
  struct Set {
    u32x4_t c[2][CL];
    uint32_t sv[2], zb[2];
  };
  auto load = [&](Set& st, int u) {
    const uint32_t sl = (uint32_t)u / kUnitsPerSlice, ui = (uint32_t)u % kUnitsPerSlice;
    const uint32_t wsl = min((uint32_t)kSliceBytes, row_bytes - (uint32_t)kSliceBytes * sl);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int j = 0; j < CL; ++j)
        st.c[t][j] = __builtin_bit_cast(
            u32x4_t, load_stream16(tbase[t] + (size_t)16 * kSliceBytes * sl +
                                   (ln * wsl + kUnitBytes * ui + (kW4 ? 16u : 32u) * lk + 16u * j)));
    st.sv[0] = st.sv[1] = st.zb[0] = st.zb[1] = 0u;
    if constexpr (kGrouped) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        st.sv[t] = sbase[t][16 * u + ln];
        if constexpr (kW4) st.zb[t] = zbase[t][8 * u + (ln >> 1)];
      }
    }
  };

  // token groups of MB blocks of 16 rows
  for (int tb = t0; tb < t1; tb += kMoeTokens * MB) {
    const int MT = min(kMoeTokens * MB, t1 - tb);
    const uint8_t* xrow[MB];  // this lane's token in each block (rows past the group repeat its last)
#pragma unroll
    for (int b = 0; b < MB; ++b)
      xrow[b] = reinterpret_cast<const uint8_t*>(x + (size_t)(tb + min(16 * b + (int)ln, MT - 1)) * K);
    f32x4_t acc[2][MB];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int b = 0; b < MB; ++b) acc[t][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // units wu, wu + W, ...: each loads and multiplies in turn (a second operand set in
    // flight doubles the registers and halves the resident waves: measured slower on
    // MI355X, like 4 or 16 waves per workgroup)
    for (int u = wu; u < U; u += W) {
      Set st;
      load(st, u);
      // the B operands of both tiles as exact fp16 code values (q, or q - z)
      u32x4_t bo[2][4];
      if constexpr (kW4) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
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
          bo[t][0] = u32x4_t{lo[0], lo8[0], lo[1], lo8[1]};
          bo[t][1] = u32x4_t{lo[2], lo8[2], lo[3], lo8[3]};
          bo[t][2] = u32x4_t{hi[0], hi8[0], hi[1], hi8[1]};
          bo[t][3] = u32x4_t{hi[2], hi8[2], hi[3], hi8[3]};
        }
      } else {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t w0 = st.c[t][j >> 1][2 * (j & 1)], w1 = st.c[t][j >> 1][2 * (j & 1) + 1];
            bo[t][j] = u32x4_t{add_f16x2(__builtin_amdgcn_perm(0x64646464u, w0, 0x04010400u), kF16Minus1152),
                               add_f16x2(__builtin_amdgcn_perm(0x64646464u, w0, 0x04030402u), kF16Minus1152),
                               add_f16x2(__builtin_amdgcn_perm(0x64646464u, w1, 0x04010400u), kF16Minus1152),
                               add_f16x2(__builtin_amdgcn_perm(0x64646464u, w1, 0x04030402u), kF16Minus1152)};
          }
      }
#pragma unroll
      for (int b = 0; b < MB; ++b) {
        if (16 * b >= MT) break;  // wave-uniform: no token of this block
        uint4 xv[4];
        const uint4* xp = reinterpret_cast<const uint4*>(xrow[b] + 2u * (128u * (uint32_t)u + 32u * lk));
#pragma unroll
        for (int j = 0; j < 4; ++j) xv[j] = xp[j];
        F16Exact fx;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          fx.add(xv[j].x);
          fx.add(xv[j].y);
          fx.add(xv[j].z);
          fx.add(xv[j].w);
        }
        const bool exact = __builtin_amdgcn_ballot_w64(!fx.ok()) != 0;
        f32x4_t d[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        if (!exact) {
          // x in fp16 (exact here), the A operands in the order of the B operands
          u32x4_t a[4];
          if constexpr (kW4) {
            a[0] = u32x4_t{bf16x2_to_f16x2(xv[0].x), bf16x2_to_f16x2(xv[0].z), bf16x2_to_f16x2(xv[1].x),
                           bf16x2_to_f16x2(xv[1].z)};
            a[1] = u32x4_t{bf16x2_to_f16x2(xv[2].x), bf16x2_to_f16x2(xv[2].z), bf16x2_to_f16x2(xv[3].x),
                           bf16x2_to_f16x2(xv[3].z)};
            a[2] = u32x4_t{bf16x2_to_f16x2(xv[0].y), bf16x2_to_f16x2(xv[0].w), bf16x2_to_f16x2(xv[1].y),
                           bf16x2_to_f16x2(xv[1].w)};
            a[3] = u32x4_t{bf16x2_to_f16x2(xv[2].y), bf16x2_to_f16x2(xv[2].w), bf16x2_to_f16x2(xv[3].y),
                           bf16x2_to_f16x2(xv[3].w)};
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
              a[j] = u32x4_t{bf16x2_to_f16x2(xv[j].x), bf16x2_to_f16x2(xv[j].y), bf16x2_to_f16x2(xv[j].z),
                             bf16x2_to_f16x2(xv[j].w)};
          }
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int t = 0; t < 2; ++t) d[t] = mma_f16(a[j], bo[t][j], d[t]);
        } else {
          // exact codes (q, or q - z) in bf16 against bf16 x
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            if constexpr (kW4) {
              const float z = (float)((st.zb[t] >> zshift) & 15u);
              auto ex = [&](uint32_t w, int i) {
                return pack_bf16x2((float)((w >> (4 * i)) & 15u) - z, (float)((w >> (16 + 4 * i)) & 15u) - z);
              };
              const uint32_t w0 = st.c[t][0][0], w1 = st.c[t][0][1], w2 = st.c[t][0][2], w3 = st.c[t][0][3];
              d[t] = mma_bf16(u32x4_t{xv[0].x, xv[0].z, xv[1].x, xv[1].z},
                              u32x4_t{ex(w0, 0), ex(w0, 2), ex(w1, 0), ex(w1, 2)}, d[t]);
              d[t] = mma_bf16(u32x4_t{xv[2].x, xv[2].z, xv[3].x, xv[3].z},
                              u32x4_t{ex(w2, 0), ex(w2, 2), ex(w3, 0), ex(w3, 2)}, d[t]);
              d[t] = mma_bf16(u32x4_t{xv[0].y, xv[0].w, xv[1].y, xv[1].w},
                              u32x4_t{ex(w0, 1), ex(w0, 3), ex(w1, 1), ex(w1, 3)}, d[t]);
              d[t] = mma_bf16(u32x4_t{xv[2].y, xv[2].w, xv[3].y, xv[3].w},
                              u32x4_t{ex(w2, 1), ex(w2, 3), ex(w3, 1), ex(w3, 3)}, d[t]);
            } else {
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                uint32_t b0, b1, b2, b3;
                i8_word_to_bf16(st.c[t][j >> 1][2 * (j & 1)], b0, b1);
                i8_word_to_bf16(st.c[t][j >> 1][2 * (j & 1) + 1], b2, b3);
                d[t] = mma_bf16(u32x4_t{xv[j].x, xv[j].y, xv[j].z, xv[j].w}, u32x4_t{b0, b1, b2, b3}, d[t]);
              }
            }
          }
        }
        // the unit's partial sums: times the group scale (group-128), or kept whole
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          if constexpr (kGrouped) {
            const float s = kW4 ? f16_to_f32((uint16_t)st.sv[t]) : bf16_to_f32((uint16_t)st.sv[t]);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[t][b][i] = fmaf(s, d[t][i], acc[t][b][i]);
          } else {
            acc[t][b] += d[t];
          }
        }
      }
    }
    // the waves' sums meet in LDS, block by block; lane l holds D[token 4 (l / 16) + i][row
    // l % 16] of both tiles
#pragma unroll
    for (int b = 0; b < MB; ++b) {
      const int tbb = tb + 16 * b, MB16 = min(16, MT - 16 * b);
      if (MB16 <= 0) break;  // uniform over the workgroup
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[((wave * 2 + t) * kMoeTokens + 4 * lk + i) * 16 + ln] = acc[t][b][i];
      __syncthreads();
      for (int o = threadIdx.x; o < (GATED ? 1 : 2) * kMoeTokens * 16; o += blockDim.x) {
        const int t = o / (kMoeTokens * 16), m = (o / 16) % kMoeTokens, r = o & 15;
        if (m >= MB16) continue;
        float v0 = 0.f, v1 = 0.f;
        for (int w = 0; w < W; ++w) {
          v0 += red[((w * 2 + t) * kMoeTokens + m) * 16 + r];
          if (GATED) v1 += red[((w * 2 + 1) * kMoeTokens + m) * 16 + r];
        }
        const int n0 = 16 * tt[t] + r;
        if constexpr (GATED) {
          const int n1 = 16 * tt[1] + r;
          const float g = kGrouped ? v0 : bf16_to_f32(sc[n0]) * v0;
          const float up = kGrouped ? v1 : bf16_to_f32(sc[n1]) * v1;
          const float h = g / (1.f + expf(-g)) * up;
          y[(size_t)(tbb + m) * (N / 2) + n0] = f32_to_bf16(h);
        } else {
          if (t == 1 && !second) continue;
          y[(size_t)(tbb + m) * N + n0] = f32_to_bf16(kGrouped ? v0 : bf16_to_f32(sc[n0]) * v0);
        }
      }
      __syncthreads();  // red is reused by the next block
    }
  }
}

template <int FMT>
void launch_fmt(bool gated, dim3 grid, const uint8_t* qw, const uint16_t* sc, const uint8_t* zs, size_t qs,
                size_t ss, size_t zst, const uint16_t* x, const int32_t* off, uint16_t* y, int T, int K, int N,
                int E, hipStream_t st) {
  // eight waves (measured on MI355X against 4, 16 and about three units per wave, with
  // and without a second operand set: 10-30 % faster at one or two tokens per expert)
  const int W = kMoeWaves;
  const size_t lds = (size_t)W * 2 * kMoeTokens * 16 * sizeof(float);
  // token blocks per pass over the weights, by the rows an expert holds on average: each
  // unit's codes then feed up to four 16-token blocks (the routing itself stays on the
  // device, so the average is all the host knows)
  const int64_t avg = (T + E - 1) / E;
  const int mb = avg <= kMoeTokens ? 1 : avg <= 2 * kMoeTokens ? 2 : avg <= 6 * kMoeTokens ? 4 : 8;
#define WQ_MOE(G, MBV) moe_kernel<FMT, G, MBV><<<grid, 64 * W, lds, st>>>(qw, sc, zs, qs, ss, zst, x, off, y, T, K, N)
  if (gated) {
    if (mb == 1) WQ_MOE(true, 1);
    else if (mb == 2) WQ_MOE(true, 2);
    else if (mb == 4) WQ_MOE(true, 4);
    else WQ_MOE(true, 8);
  } else {
    if (mb == 1) WQ_MOE(false, 1);
    else if (mb == 2) WQ_MOE(false, 2);
    else if (mb == 4) WQ_MOE(false, 4);
    else WQ_MOE(false, 8);
  }
#undef WQ_MOE
}

}  // namespace

wq_status launch_moe(const wq_weight* w, int E, const uint16_t* x, const int32_t* offsets, int64_t T, uint16_t* y,
                     bool gated, size_t qw_stride, size_t sc_stride, size_t zs_stride, hipStream_t s) {
  const int T16 = (int)(w->N / 16);
  const dim3 grid((unsigned)(gated ? T16 / 2 : (T16 + 1) / 2), (unsigned)E);
  const uint8_t* qw = (const uint8_t*)w->qweight;
  const uint16_t* sc = (const uint16_t*)w->scales;
  const uint8_t* zs = (const uint8_t*)w->zeros;
  switch (w->fmt) {
    case WQ_FMT_W8_PC:
      launch_fmt<WQ_FMT_W8_PC>(gated, grid, qw, sc, zs, qw_stride, sc_stride, zs_stride, x, offsets, y, (int)T,
                               (int)w->K, (int)w->N, E, s);
      break;
    case WQ_FMT_W8_G128:
      launch_fmt<WQ_FMT_W8_G128>(gated, grid, qw, sc, zs, qw_stride, sc_stride, zs_stride, x, offsets, y, (int)T,
                                 (int)w->K, (int)w->N, E, s);
      break;
    case WQ_FMT_W4_G128:
      launch_fmt<WQ_FMT_W4_G128>(gated, grid, qw, sc, zs, qw_stride, sc_stride, zs_stride, x, offsets, y, (int)T,
                                 (int)w->K, (int)w->N, E, s);
      break;
    default:
      return fail(WQ_ERR_UNSUPPORTED, "wq_moe_linear: unknown format");
  }
  WQ_HIP_CHECK(hipGetLastError());
  return WQ_OK;
}

}  // namespace wq
