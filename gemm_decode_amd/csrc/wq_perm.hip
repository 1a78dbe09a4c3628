// Full-K activation permutation (act-order): the layer's weight is stored with its K
// columns in a permuted order, so that the quantisation groups are contiguous in
// storage, and the activations are gathered by the same index before the product:
// x'[m][j] = x[m][perm[j]], then y = x' . dequant(W)^T.  The Marlin register and
// launch scheduling benchmark page lists the full-K activation permutation among the
// validated cases ("Validation and limits") and counts activation-order index
// storage in the dense kernel's shared memory; the gather here is a pre-pass into
// the workspace, after which the ordinary GEMV / GEMM path runs unchanged.
#include "wq_internal.h"

namespace wq {
namespace {

// One thread per 8 consecutive outputs of a row: 8 index loads (two 16-byte loads
// when the index array is 16-byte aligned), 8 gathered 2-byte reads of x (the row
// stays in L2: at most 8 MB for the largest K), one 16-byte store.  An index outside
// [0, K) reads as +0.
template <bool kVecIdx>
__global__ __launch_bounds__(256) void perm_gather_kernel(const uint16_t* __restrict__ x,
                                                          const int32_t* __restrict__ perm,
                                                          uint16_t* __restrict__ xp, int64_t M, int K) {
  const int64_t per_row = K / 8;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= M * per_row) return;
  const int64_t m = i / per_row;
  const int j0 = (int)(i - m * per_row) * 8;
  int idx[8];
  if constexpr (kVecIdx) {
    const int4 a = *reinterpret_cast<const int4*>(perm + j0), b = *reinterpret_cast<const int4*>(perm + j0 + 4);
    idx[0] = a.x; idx[1] = a.y; idx[2] = a.z; idx[3] = a.w;
    idx[4] = b.x; idx[5] = b.y; idx[6] = b.z; idx[7] = b.w;
  } else {
#pragma unroll
    for (int t = 0; t < 8; ++t) idx[t] = perm[j0 + t];
  }
  const uint16_t* xr = x + m * K;
  uint32_t v[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) v[t] = ((unsigned)idx[t] < (unsigned)K) ? xr[idx[t]] : 0u;
  uint4 o;
  o.x = v[0] | (v[1] << 16);
  o.y = v[2] | (v[3] << 16);
  o.z = v[4] | (v[5] << 16);
  o.w = v[6] | (v[7] << 16);
  *reinterpret_cast<uint4*>(xp + m * K + j0) = o;
}

// Row-staged form for large M: one workgroup per token row copies the row of x into
// LDS with 16-byte loads, then gathers from LDS and writes x' with 16-byte stores, so
// HBM sees x and x' once each, coalesced.  K * 2 bytes of LDS (K <= kStagedMaxK).
constexpr int kStagedMaxK = 32768;
__global__ __launch_bounds__(1024) void perm_gather_row_kernel(const uint16_t* __restrict__ x,
                                                               const int32_t* __restrict__ perm,
                                                               uint16_t* __restrict__ xp, int K) {
  __shared__ uint4 row[kStagedMaxK / 8];
  const int64_t m = blockIdx.x;
  const uint4* xr = reinterpret_cast<const uint4*>(x + m * K);
  const int n8 = K / 8;
  for (int i = threadIdx.x; i < n8; i += blockDim.x) row[i] = xr[i];
  __syncthreads();
  const uint16_t* rs = reinterpret_cast<const uint16_t*>(row);
  uint4* out = reinterpret_cast<uint4*>(xp + m * K);
  for (int i = threadIdx.x; i < n8; i += blockDim.x) {
    const int4 a = reinterpret_cast<const int4*>(perm)[2 * i], b = reinterpret_cast<const int4*>(perm)[2 * i + 1];
    const int idx[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    uint32_t v[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) v[t] = ((unsigned)idx[t] < (unsigned)K) ? rs[idx[t]] : 0u;
    uint4 o;
    o.x = v[0] | (v[1] << 16);
    o.y = v[2] | (v[3] << 16);
    o.z = v[4] | (v[5] << 16);
    o.w = v[6] | (v[7] << 16);
    out[i] = o;
  }
}

}  // namespace

wq_status launch_perm_gather(const uint16_t* x, const int32_t* perm, uint16_t* xp, int64_t M, int64_t K,
                             hipStream_t s) {
  // many rows, 16-byte aligned x and indices, a row that fits in LDS: the row-staged form
  if (M >= 64 && K <= kStagedMaxK && (uintptr_t)x % 16 == 0 && (uintptr_t)perm % 16 == 0) {
    if (M > INT32_MAX) return fail(WQ_ERR_UNSUPPORTED, "activation gather: M too large");
    perm_gather_row_kernel<<<(unsigned)M, 1024, 0, s>>>(x, perm, xp, (int)K);
    WQ_HIP_CHECK(hipGetLastError());
    return WQ_OK;
  }
  const int64_t threads = M * (K / 8);
  const int64_t blocks = (threads + 255) / 256;
  if (blocks > INT32_MAX) return fail(WQ_ERR_UNSUPPORTED, "activation gather: M * K too large");
  if ((uintptr_t)perm % 16 == 0)
    perm_gather_kernel<true><<<(unsigned)blocks, 256, 0, s>>>(x, perm, xp, M, (int)K);
  else
    perm_gather_kernel<false><<<(unsigned)blocks, 256, 0, s>>>(x, perm, xp, M, (int)K);
  WQ_HIP_CHECK(hipGetLastError());
  return WQ_OK;
}

}  // namespace wq
