// Routing kernels: top-k selection with softmax-renormalised weights (one wavefront per
// token) and the per-chunk expert histogram of a whole prompt.
#include <math.h>

#include <algorithm>

#include "device_common.h"
#include "moe_internal.h"
#include "profile.h"
#include "topk_select.h"

namespace moe {
namespace {

// Lane `lane`'s logits of token t: experts lane*NJ .. lane*NJ+NJ-1, -inf past E or T. 16-byte
// loads where all of them exist and their address is 16-byte aligned.
template <int NJ>
__device__ __forceinline__ void load_logits(const float* __restrict__ logits, int64_t T, int E,
                                            int64_t t, int lane, float (&x)[NJ]) {
  const int64_t off = t * E + static_cast<int64_t>(lane) * NJ;
  if constexpr (NJ % 4 == 0) {
    if (t < T && lane * NJ + NJ <= E && (reinterpret_cast<uintptr_t>(logits + off) & 15) == 0) {
#pragma unroll
      for (int q = 0; q < NJ / 4; ++q) {
        const f32x4_t v = *reinterpret_cast<const f32x4_t*>(logits + off + 4 * q);
        x[4 * q] = v[0];
        x[4 * q + 1] = v[1];
        x[4 * q + 2] = v[2];
        x[4 * q + 3] = v[3];
      }
      return;
    }
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j)
    x[j] = (t < T && lane * NJ + j < E) ? logits[off + j] : -INFINITY;
}

// One wavefront per token (topk_select); lane l loads the logits of experts l*NJ .. l*NJ+NJ-1.
// The kernel also zeroes n_zero ints at `zero` (the per-chunk counts the next kernel adds
// to), so that needs no launch of its own.
template <int NJ>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int64_t T,
                                                   int E, int k, int32_t* __restrict__ ids,
                                                   float* __restrict__ weights,
                                                   int32_t* __restrict__ zero, int64_t n_zero) {
  __shared__ uint64_t lst[4][topk_lds_words<NJ>()];
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n_zero;
       i += static_cast<int64_t>(gridDim.x) * 256)
    zero[i] = 0;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + wv;
  float x[NJ];
  load_logits<NJ>(logits, T, E, t, lane, x);
  topk_select<NJ>(x, E, k, t < T, ids + t * k, weights + t * k, lst[wv]);
}

// A prompt of at most 16 tokens in one workgroup: one wavefront per token as above, then the
// same workgroup zeroes the per-chunk counts and adds every slot to them (one launch instead
// of two; integer counts, so the order of the adds is free).
constexpr int kSmallTopkTokens = 16;
template <int NJ>
__global__ __launch_bounds__(64 * kSmallTopkTokens) void topk_counts_small_kernel(
    const float* __restrict__ logits, int64_t T, int E, int k, int32_t* __restrict__ ids,
    float* __restrict__ weights, int64_t chunk, int32_t* __restrict__ cc, int64_t n_cc) {
  __shared__ uint64_t lst[kSmallTopkTokens][topk_lds_words<NJ>()];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t t = wv;
  float x[NJ];
  load_logits<NJ>(logits, T, E, t, lane, x);
  topk_select<NJ>(x, E, k, t < T, ids + t * k, weights + t * k, lst[wv]);
  for (int64_t i = threadIdx.x; i < n_cc; i += blockDim.x) cc[i] = 0;
  __syncthreads();              // ids written and counts zeroed, for the whole workgroup
  for (int64_t i = threadIdx.x; i < T * k; i += blockDim.x)
    atomicAdd(&cc[(i / k / chunk) * E + ids[i]], 1);
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
                       float* weights, int32_t* zero, int64_t n_zero, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  ProfScope prof(MOE_STAGE_TOPK, s);
  const unsigned blocks = static_cast<unsigned>((T + 3) / 4);
  const int nj = (E + 63) / 64;
  if (nj <= 1) topk_kernel<1><<<blocks, 256, 0, s>>>(logits, T, E, k, ids, weights, zero, n_zero);
  else if (nj <= 2) topk_kernel<2><<<blocks, 256, 0, s>>>(logits, T, E, k, ids, weights, zero, n_zero);
  else if (nj <= 4) topk_kernel<4><<<blocks, 256, 0, s>>>(logits, T, E, k, ids, weights, zero, n_zero);
  else if (nj <= 8) topk_kernel<8><<<blocks, 256, 0, s>>>(logits, T, E, k, ids, weights, zero, n_zero);
  else topk_kernel<16><<<blocks, 256, 0, s>>>(logits, T, E, k, ids, weights, zero, n_zero);
  return hipGetLastError();
}

bool topk_counts_fused(int64_t T) { return T > 0 && T <= kSmallTopkTokens; }

hipError_t launch_topk_counts_small(const float* logits, int64_t T, int E, int k, int32_t* ids,
                                    float* weights, int64_t chunk, int32_t* chunk_counts,
                                    int64_t n_cc, hipStream_t s) {
  if (!topk_counts_fused(T)) return hipErrorInvalidValue;
  ProfScope prof(MOE_STAGE_TOPK, s);
  const unsigned threads = static_cast<unsigned>(64 * T);
  const int nj = (E + 63) / 64;
  if (nj <= 1) topk_counts_small_kernel<1><<<1, threads, 0, s>>>(logits, T, E, k, ids, weights, chunk, chunk_counts, n_cc);
  else if (nj <= 2) topk_counts_small_kernel<2><<<1, threads, 0, s>>>(logits, T, E, k, ids, weights, chunk, chunk_counts, n_cc);
  else if (nj <= 4) topk_counts_small_kernel<4><<<1, threads, 0, s>>>(logits, T, E, k, ids, weights, chunk, chunk_counts, n_cc);
  else if (nj <= 8) topk_counts_small_kernel<8><<<1, threads, 0, s>>>(logits, T, E, k, ids, weights, chunk, chunk_counts, n_cc);
  else topk_counts_small_kernel<16><<<1, threads, 0, s>>>(logits, T, E, k, ids, weights, chunk, chunk_counts, n_cc);
  return hipGetLastError();
}

hipError_t launch_chunk_hist(const int32_t* ids, int64_t T, int k, int E, int64_t chunk,
                             int32_t* chunk_counts, hipStream_t s) {
  ProfScope prof(MOE_STAGE_CHUNK_COUNTS, s);
  if (T <= 0) return hipSuccess;      // chunk_counts were zeroed by the top-k kernel
  chunk_hist_kernel<<<static_cast<unsigned>((T + 255) / 256), 256, 0, s>>>(ids, T, k, E, chunk,
                                                                           chunk_counts);
  return hipGetLastError();
}

}  // namespace moe
