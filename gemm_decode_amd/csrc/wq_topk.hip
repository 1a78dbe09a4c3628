// LM head + top-k sampling: after the layer has written bf16 logits [M][V] (the
// GEMV for decode, into the workspace), two kernels pick the k best logits of every
// row and draw one token from them ("Fused LM Head + Top-k" and "Distributed Top-k
// Sampling" in the tileInfer README's feature list: logits and sampling in one step,
// and only the k best logits leave their producer).
//
// Order: larger value first, equal values by smaller index, -0 == +0, NaN after
// every number.  A logit's rank value is an order-preserving 16-bit map of its bf16
// bits (NaN -> 0, below every number) with bit 16 set; empty slots rank 0, below all.
//
//   topk_chunk_kernel         grid (ceil(V / 2048), M), 256 threads x 8 logits: the
//                             chunk's k best (index ties by position) -> workspace;
//   topk_merge_sample_kernel  grid M, 1024 threads x 8 candidates: the row's k best
//                             of the chunk candidates (each carries its logit's
//                             bits) and the drawn token.
//
// Selection, in two wave-level stages without block-wide searches: every wave keeps
// the k best of its 512 entries (wave_select: a search over the rank, three ballot
// counts per step, then ballot prefix counts give each kept entry a slot), then wave 0
// (through four waves first in the merge kernel) keeps the k best of the waves' lists
// and orders them (each kept key's place is its count of better kept keys).  A key holds the rank, then the complemented index (so
// equal ranks order by index), then the logit's own bits.
//
// Sampling (one wave, lane i holds the i-th best): weights exp((v_i - v_1) / T) in
// fp32, an inclusive scan across the lanes, token = the first lane whose running sum
// exceeds u * total (the last kept one if none does); temperature 0 or a non-finite
// best logit takes the best; a NaN logit behind a finite best weighs 0.
#include "wq_internal.h"

namespace wq {
namespace {

constexpr int kTopkChunk = 2048;
constexpr int kTopkPer = 8;  // entries per thread (consecutive positions)

__device__ __forceinline__ uint32_t topk_rank(uint16_t h) {
  const uint32_t b = (h & 0x7FFFu) ? h : 0u;                                 // -0 == +0
  const uint32_t ord = (b & 0x8000u) ? (~b & 0xFFFFu) : (b | 0x8000u);
  const bool nan = (b & 0x7FFFu) > 0x7F80u;                                  // NaN: below every number
  return 0x10000u | (nan ? 0u : ord);
}

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Keys: rank (17 bits) | ~index (31 bits) | the logit's own bf16 bits (16): larger is
// better, equal ranks order by index, and the bits travel with the entry.
__device__ __forceinline__ uint64_t topk_key(uint32_t rank, uint32_t index, uint16_t bits) {
  return ((uint64_t)rank << 47) | ((uint64_t)(0x7FFFFFFFu - index) << 16) | bits;
}
__device__ __forceinline__ uint32_t key_rank(uint64_t key) { return (uint32_t)(key >> 47); }
__device__ __forceinline__ uint32_t key_index(uint64_t key) { return 0x7FFFFFFFu - (uint32_t)((key >> 16) & 0x7FFFFFFFu); }
__device__ __forceinline__ uint16_t key_bits(uint64_t key) { return (uint16_t)key; }

// One wave keeps the k best of its 64 x E keys (rank 0 = empty slot).  Entries of equal rank must lie in index order along the lane-major
// positions lane * E + j; k <= the wave's nonempty entries, k <= 64.  Writes the kept
// keys to dst[0 .. k) in no particular order.  Control flow is wave-uniform: a binary
// search over the rank finds the k-th best rank T from ballot counts; the entries
// above T and the first k - #above entries at T (position order, from ballot prefix
// counts) take the k slots.
template <int E>
__device__ __forceinline__ uint32_t wave_count_ge(const uint64_t (&key)[E], uint32_t v) {
  uint32_t c = 0;
#pragma unroll
  for (int j = 0; j < E; ++j) c += (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(key_rank(key[j]) >= v));
  return c;
}

template <int E>
__device__ void wave_select(const uint64_t (&key)[E], int k, uint64_t* dst) {
  // invariant: #(rank >= lo) >= k > #(rank >= hi); three thresholds per step (the
  // counts are independent, so their latencies overlap), then halving for the rest
  uint32_t lo = 0, hi = 1u << 17;
  while (hi - lo >= 4) {
    const uint32_t q = (hi - lo) >> 2, t1 = lo + q, t2 = lo + 2 * q, t3 = lo + 3 * q;
    const uint32_t c1 = wave_count_ge(key, t1), c2 = wave_count_ge(key, t2), c3 = wave_count_ge(key, t3);
    if (c3 >= (uint32_t)k) {
      lo = t3;
    } else if (c2 >= (uint32_t)k) {
      lo = t2;
      hi = t3;
    } else if (c1 >= (uint32_t)k) {
      lo = t1;
      hi = t2;
    } else {
      hi = t1;
    }
  }
  while (hi - lo > 1) {
    const uint32_t mid = (lo + hi) >> 1;
    if (wave_count_ge(key, mid) >= (uint32_t)k) lo = mid;
    else hi = mid;
  }
  const uint32_t T = lo;
  uint32_t gt_below = 0, eq_below = 0, tg = 0;
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const uint32_t r = key_rank(key[j]);
    const uint64_t mg = __builtin_amdgcn_ballot_w64(r > T), me = __builtin_amdgcn_ballot_w64(r == T);
    gt_below += lanes_below(mg);
    eq_below += lanes_below(me);
    tg += (uint32_t)__builtin_popcountll(mg);
  }
  const uint32_t need = (uint32_t)k - tg;
  uint32_t og = gt_below, oe = eq_below;
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const uint32_t r = key_rank(key[j]);
    if (r > T) {
      dst[og++] = key[j];
    } else if (r == T) {
      if (oe < need) dst[tg + oe] = key[j];
      ++oe;
    }
  }
}

// One wave: src[0 .. k) (distinct nonzero keys, src[k .. 64) zero) -> dst[0 .. k) best
// first; each kept key's place is its count of better keys (two keys per LDS read, all
// reads issued before the compares).
__device__ __forceinline__ void wave_rank_sort(const uint64_t* src, int k, uint64_t* dst) {
  const int lane = threadIdx.x & 63;
  const uint64_t own = src[lane];
  const ulonglong2* s2 = reinterpret_cast<const ulonglong2*>(src);
  ulonglong2 all[32];
#pragma unroll
  for (int j = 0; j < 32; ++j) all[j] = s2[j];
  int pos = 0;
#pragma unroll
  for (int j = 0; j < 32; ++j) pos += (all[j].x > own ? 1 : 0) + (all[j].y > own ? 1 : 0);
  if (lane < k) dst[pos] = own;
}

// One wave: the k best (fewer if the lists hold fewer) of the NL lists lists[w][0 .. 64)
// (empty slots 0), read lane-major so that list order (= index order for equal ranks)
// is position order; writes them to dst[0 .. kept) unordered and zeros the rest of
// dst[0 .. 64); returns kept.
template <int NL>
__device__ int select_lists(const uint64_t (*lists)[64], int k, uint64_t* dst) {
  constexpr int E = NL;  // 64 x NL entries over 64 lanes
  const int lane = threadIdx.x & 63;
  const uint64_t* flat = &lists[0][0];
  uint64_t key[E];
  uint32_t nonempty = 0;
#pragma unroll
  for (int j = 0; j < E; ++j) {
    key[j] = flat[lane * E + j];
    nonempty += (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(key[j] != 0ull));
  }
  const int kept = min(k, (int)nonempty);
  if (lane >= kept) dst[lane] = 0ull;  // (the same wave fills [0, kept) next)
  if (kept > 0) wave_select<E>(key, kept, dst);
  return kept;
}

__global__ __launch_bounds__(256) void topk_chunk_kernel(const uint16_t* __restrict__ logits, int V, int k,
                                                         uint64_t* __restrict__ cand) {
  constexpr int NW = 4;
  __shared__ uint64_t stage[NW][64];
  __shared__ __attribute__((aligned(16))) uint64_t tmp[64];
  __shared__ uint64_t fin[64];
  const int c = blockIdx.x, m = blockIdx.y, t = threadIdx.x, P = gridDim.x;
  const int lane = t & 63, wv = t >> 6;
  const uint16_t* row = logits + (size_t)m * V;
  const int base = c * kTopkChunk, n = min(kTopkChunk, V - base);
  // all eight loads issued before any use (a load under its own branch would wait
  // for each in turn); slots past the chunk read its last logit and rank 0
  uint16_t b[kTopkPer];
#pragma unroll
  for (int j = 0; j < kTopkPer; ++j) b[j] = row[base + min(t * kTopkPer + j, n - 1)];
  uint64_t key[kTopkPer];
#pragma unroll
  for (int j = 0; j < kTopkPer; ++j) {
    const int p = t * kTopkPer + j;
    key[j] = p < n ? topk_key(topk_rank(b[j]), (uint32_t)(base + p), b[j]) : 0ull;
  }
  const int nw = min(max(n - wv * 64 * kTopkPer, 0), 64 * kTopkPer);  // this wave's entries
  const int kw = min(k, nw);
  if (kw > 0) wave_select<kTopkPer>(key, kw, stage[wv]);
  if (lane >= kw) stage[wv][lane] = 0ull;
  __syncthreads();
  if (wv == 0) {
    const int kk = select_lists<NW>(stage, k, tmp);   // = min(k, n)
    wave_rank_sort(tmp, kk, fin);
    uint64_t* out = cand + ((size_t)m * P + c) * k;
    if (lane < k) out[lane] = lane < kk ? fin[lane] : 0ull;
  }
}

__global__ __launch_bounds__(1024) void topk_merge_sample_kernel(int k, int P, const uint64_t* __restrict__ cand,
                                                                 float temperature, const float* __restrict__ u,
                                                                 uint16_t* __restrict__ top_vals,
                                                                 int32_t* __restrict__ top_idx,
                                                                 int32_t* __restrict__ tokens) {
  constexpr int NW = 16;
  __shared__ uint64_t stage[NW][64];
  __shared__ uint64_t part[4][64];
  __shared__ __attribute__((aligned(16))) uint64_t tmp[64];
  __shared__ uint64_t fin[64];
  const int m = blockIdx.x, t = threadIdx.x;
  const int lane = t & 63, wv = t >> 6;
  const int n = P * k;  // <= 8192 = 1024 x 8 (checked on the host)
  const uint64_t* row = cand + (size_t)m * n;
  uint64_t key[kTopkPer];
#pragma unroll
  for (int j = 0; j < kTopkPer; ++j) key[j] = row[min(t * kTopkPer + j, n - 1)];  // loads first
  uint32_t nonempty = 0;
#pragma unroll
  for (int j = 0; j < kTopkPer; ++j) {
    if (t * kTopkPer + j >= n) key[j] = 0ull;
    nonempty += (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(key[j] != 0ull));
  }
  const int kw = min(k, (int)nonempty);
  if (kw > 0) wave_select<kTopkPer>(key, kw, stage[wv]);
  if (lane >= kw) stage[wv][lane] = 0ull;
  __syncthreads();
  // 16 lists -> 4 (waves 0-3, four lists each) -> 1 (wave 0), then ordered
  if (wv < 4) select_lists<4>(&stage[4 * wv], k, part[wv]);
  __syncthreads();
  if (wv != 0) return;
  select_lists<4>(part, k, tmp);
  wave_rank_sort(tmp, k, fin);
  // wave 0: lane i holds the i-th best (k <= 64)
  const bool live = lane < k;
  const uint64_t best = live ? fin[lane] : 0ull;
  const uint32_t idx = key_index(best);
  const uint16_t bits = key_bits(best);
  if (live) {
    top_idx[(size_t)m * k + lane] = (int32_t)idx;
    top_vals[(size_t)m * k + lane] = bits;
  }
  const float v = __uint_as_float((uint32_t)bits << 16);
  const float v1 = __shfl(v, 0);
  const float w = (live && !__builtin_isnan(v)) ? expf((v - v1) / temperature) : 0.f;
  float run = w;
  for (int d = 1; d < 64; d <<= 1) {
    const float o = __shfl_up(run, d);
    if (lane >= d) run += o;
  }
  const float total = __shfl(run, k - 1);
  const float thr = u[m] * total;
  const uint64_t hit = __builtin_amdgcn_ballot_w64(live && run > thr);
  const int pick = hit ? __builtin_ctzll(hit) : k - 1;
  const uint32_t tok = __shfl((int)idx, pick);
  if (lane == 0) {
    const bool greedy = temperature == 0.f || !__builtin_isfinite(v1);
    tokens[m] = (int32_t)(greedy ? idx : tok);
  }
}

}  // namespace

int topk_chunks(int64_t V) { return (int)((V + kTopkChunk - 1) / kTopkChunk); }

wq_status launch_topk(const uint16_t* logits, int64_t M, int64_t V, int k, float temperature, const float* u,
                      uint64_t* cand, uint16_t* top_vals, int32_t* top_idx, int32_t* tokens, hipStream_t s) {
  const int P = topk_chunks(V);
  topk_chunk_kernel<<<dim3((unsigned)P, (unsigned)M), 256, 0, s>>>(logits, (int)V, k, cand);
  WQ_HIP_CHECK(hipGetLastError());
  topk_merge_sample_kernel<<<(unsigned)M, 1024, 0, s>>>(k, P, cand, temperature, u, top_vals, top_idx, tokens);
  WQ_HIP_CHECK(hipGetLastError());
  return WQ_OK;
}

}  // namespace wq
