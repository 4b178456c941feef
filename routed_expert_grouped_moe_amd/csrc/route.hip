// Routing kernels: top-k selection with softmax-renormalised weights (one wavefront per
// token) and the per-chunk expert histogram of a whole prompt.
#include <math.h>

#include <algorithm>

#include "device_common.h"
#include "moe_internal.h"
#include "profile.h"

namespace moe {
namespace {

// Orderable 32-bit key of a float: a > b as floats (no NaN) iff key(a) > key(b) as unsigned.
// Every key of a real value is above 0x007FFFFF (the key of -inf); 0 marks a taken or missing
// entry.
__device__ __forceinline__ uint32_t order_key(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

// Wavefront maximum of an unsigned key with DPP moves: within quads, mirrored half rows and
// rows, then row broadcasts; the result is valid in lane 63.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ uint32_t dpp_max_step(uint32_t m) {
  const uint32_t o = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(
      static_cast<int>(m), static_cast<int>(m), kCtrl, kRowMask, 0xF, false));
  return o > m ? o : m;
}
__device__ __forceinline__ uint32_t wave_max(uint32_t m) {
  m = dpp_max_step<0xB1, 0xF>(m);     // quad_perm [1,0,3,2]
  m = dpp_max_step<0x4E, 0xF>(m);     // quad_perm [2,3,0,1]
  m = dpp_max_step<0x141, 0xF>(m);    // row_half_mirror
  m = dpp_max_step<0x140, 0xF>(m);    // row_mirror
  m = dpp_max_step<0x142, 0xA>(m);    // row_bcast:15 into rows 1 and 3
  m = dpp_max_step<0x143, 0xC>(m);    // row_bcast:31 into rows 2 and 3
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(m), 63));
}

// One wavefront per token; lane l holds the logits of experts l, l + 64, ..., l + 64 (NJ-1).
// k rounds pick the k largest logits, the lower id among equal values, NaN ranking as -inf
// (and -0 as +0): a round takes the wavefront maximum of the untaken keys, then the lowest id
// holding it (the first 64-expert slice with a match, its lowest lane, by ballots). The chosen
// ids are written in ascending order by a ballot compaction, and each weight is
// exp(l - l_max) / (sum over the chosen of exp(l' - l_max), taken in ascending id), which
// equals the softmax over all experts renormalised over the chosen ones.
template <int NJ>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int64_t T,
                                                   int E, int k, int32_t* __restrict__ ids,
                                                   float* __restrict__ weights) {
  __shared__ float ex[4][1024];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + wv;
  const bool active = t < T;

  float v[NJ];
  uint32_t key[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int e = lane + 64 * j;
    float x = -INFINITY;
    if (active && e < E) x = logits[t * E + e];
    if (x != x) x = -INFINITY;
    if (x == 0.f) x = 0.f;     // -0 and +0 are equal logits: one key for both
    v[j] = x;
    key[j] = e < E ? order_key(x) : 0u;
  }
  uint32_t taken = 0;
  float vmax = 0.f;
  for (int r = 0; r < k; ++r) {
    uint32_t m = key[0];
#pragma unroll
    for (int j = 1; j < NJ; ++j) m = key[j] > m ? key[j] : m;
    const uint32_t best = wave_max(m);
    int jw = 0, lw = 0;
#pragma unroll
    for (int j = NJ - 1; j >= 0; --j) {   // ends at the lowest slice holding the maximum
      const uint64_t b = __ballot(key[j] == best);
      if (b) {
        jw = j;
        lw = __ffsll(static_cast<unsigned long long>(b)) - 1;
      }
    }
    if (r == 0) vmax = key_value(best);
    if (lane == lw) {
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        if (j == jw) {
          key[j] = 0u;
          taken |= 1u << j;
        }
    }
  }
  int base = 0;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const bool tk = (taken >> j) & 1u;
    const uint64_t m = __ballot(tk);
    if (tk) {
      const int pos = base + __popcll(m & ((1ull << lane) - 1ull));
      if (active) ids[t * k + pos] = lane + 64 * j;
      ex[wv][pos] = v[j];
    }
    base += __popcll(m);
  }
  __syncthreads();
  for (int p = lane; p < k; p += 64) ex[wv][p] = expf(ex[wv][p] - vmax);
  __syncthreads();
  float sum = 0.f;
  if (lane == 0)
    for (int p = 0; p < k; ++p) sum += ex[wv][p];
  sum = __shfl(sum, 0);
  if (active)
    for (int p = lane; p < k; p += 64) weights[t * k + p] = ex[wv][p] / sum;
}

// Per-chunk expert counts. Block b covers tokens [256 b, 256 b + 256); when the chunks it
// spans fit an LDS histogram it counts there and adds each nonzero bin to the global counts
// once, else it adds every slot directly. Integer counts, so the order of the adds is free.
constexpr int kHistBins = 4096;
__global__ __launch_bounds__(256) void chunk_hist_kernel(const int32_t* __restrict__ ids,
                                                         int64_t T, int k, int E, int64_t chunk,
                                                         int32_t* __restrict__ cc) {
  __shared__ int32_t hist[kHistBins];
  const int tid = threadIdx.x;
  const int64_t t_lo = static_cast<int64_t>(blockIdx.x) * 256;
  const int64_t t_hi = t_lo + 256 < T ? t_lo + 256 : T;
  const int64_t c_lo = t_lo / chunk, c_hi = (t_hi - 1) / chunk;
  const int64_t bins = (c_hi - c_lo + 1) * E;
  if (bins > kHistBins) {
    for (int64_t i = t_lo * k + tid; i < t_hi * k; i += 256)
      atomicAdd(&cc[(i / k / chunk) * E + ids[i]], 1);
    return;
  }
  for (int b = tid; b < bins; b += 256) hist[b] = 0;
  __syncthreads();
  for (int64_t i = t_lo * k + tid; i < t_hi * k; i += 256)
    atomicAdd(&hist[(i / k / chunk - c_lo) * E + ids[i]], 1);
  __syncthreads();
  for (int b = tid; b < bins; b += 256)
    if (hist[b]) atomicAdd(&cc[c_lo * E + b], hist[b]);
}

__global__ void fill_i32_kernel(int32_t* p, int64_t n, int32_t v) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * 256)
    p[i] = v;
}

}  // namespace

hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
  fill_i32_kernel<<<static_cast<unsigned>(blocks), 256, 0, s>>>(p, n, v);
  return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int64_t T, int E, int k, int32_t* ids,
                       float* weights, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  ProfScope prof(MOE_STAGE_TOPK, s);
  const unsigned blocks = static_cast<unsigned>((T + 3) / 4);
  const int nj = (E + 63) / 64;
  if (nj <= 1) topk_kernel<1><<<blocks, 256, 0, s>>>(logits, T, E, k, ids, weights);
  else if (nj <= 2) topk_kernel<2><<<blocks, 256, 0, s>>>(logits, T, E, k, ids, weights);
  else if (nj <= 4) topk_kernel<4><<<blocks, 256, 0, s>>>(logits, T, E, k, ids, weights);
  else if (nj <= 8) topk_kernel<8><<<blocks, 256, 0, s>>>(logits, T, E, k, ids, weights);
  else topk_kernel<16><<<blocks, 256, 0, s>>>(logits, T, E, k, ids, weights);
  return hipGetLastError();
}

hipError_t launch_chunk_hist(const int32_t* ids, int64_t T, int k, int E, int64_t chunk,
                             int32_t* chunk_counts, hipStream_t s) {
  const int64_t n_chunks = (T + chunk - 1) / chunk;
  ProfScope prof(MOE_STAGE_CHUNK_COUNTS, s);
  hipError_t err = launch_fill_i32(chunk_counts, n_chunks * E, 0, s);
  if (err != hipSuccess || T <= 0) return err;
  chunk_hist_kernel<<<static_cast<unsigned>((T + 255) / 256), 256, 0, s>>>(ids, T, k, E, chunk,
                                                                           chunk_counts);
  return hipGetLastError();
}

}  // namespace moe
