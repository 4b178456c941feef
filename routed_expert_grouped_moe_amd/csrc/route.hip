// Routing kernels: top-k selection with softmax-renormalised weights (one wavefront per
// token) and the per-chunk expert histogram of a whole prompt.
#include <math.h>

#include <algorithm>

#include "device_common.h"
#include "moe_internal.h"
#include "profile.h"

namespace moe {
namespace {

constexpr int kMaxLanes = 16;   // logits per lane: E <= 1024 = 16 * 64

// a "better" (value, id) pair: larger value, or equal value and lower id
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

// One wavefront per token. Lane l holds logits of experts l, l + 64, ... . k rounds of a wave
// argmax pick the k largest (lower id on equal values; NaN ranks as -inf); the chosen ids are
// then written in ascending order by a ballot compaction, and each weight is
// exp(l - l_max) / sum over the chosen of exp(l' - l_max), the sum taken in ascending id.
// This equals the softmax over all experts renormalised over the chosen ones.
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int64_t T,
                                                   int E, int k, int32_t* __restrict__ ids,
                                                   float* __restrict__ weights) {
  __shared__ float ex[4][1024];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + wv;
  const bool active = t < T;
  const int nj = (E + 63) / 64;

  float v[kMaxLanes];
#pragma unroll
  for (int j = 0; j < kMaxLanes; ++j) {
    const int e = lane + 64 * j;
    float x = -INFINITY;
    if (active && j < nj && e < E) x = logits[t * E + e];
    v[j] = (x != x) ? -INFINITY : x;
  }
  uint32_t taken = 0;
  float vmax = 0.f;
  for (int r = 0; r < k; ++r) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < kMaxLanes; ++j) {
      const int e = lane + 64 * j;
      if (j < nj && e < E && !((taken >> j) & 1u) && better(v[j], e, bv, bi)) {
        bv = v[j];
        bi = e;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      if (better(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (r == 0) vmax = bv;
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
  }
  int base = 0;
#pragma unroll
  for (int j = 0; j < kMaxLanes; ++j) {
    const bool tk = j < nj && ((taken >> j) & 1u);
    const uint64_t m = __ballot(tk);
    if (tk) {
      const int pos = base + __popcll(m & ((1ull << lane) - 1ull));
      if (active) ids[t * k + pos] = lane + 64 * j;
      ex[wv][pos] = expf(v[j] - vmax);
    }
    base += __popcll(m);
  }
  __syncthreads();
  float sum = 0.f;
  if (lane == 0)
    for (int p = 0; p < k; ++p) sum += ex[wv][p];
  sum = __shfl(sum, 0);
  if (active)
    for (int p = lane; p < k; p += 64) weights[t * k + p] = ex[wv][p] / sum;
}

__global__ void chunk_hist_kernel(const int32_t* __restrict__ ids, int64_t slots, int k, int E,
                                  int64_t chunk, int32_t* __restrict__ cc) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= slots) return;
  const int64_t t = i / k;
  atomicAdd(&cc[(t / chunk) * E + ids[i]], 1);   // integer counts: order-free
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
  topk_kernel<<<static_cast<unsigned>((T + 3) / 4), 256, 0, s>>>(logits, T, E, k, ids, weights);
  return hipGetLastError();
}

hipError_t launch_chunk_hist(const int32_t* ids, int64_t T, int k, int E, int64_t chunk,
                             int32_t* chunk_counts, hipStream_t s) {
  const int64_t n_chunks = (T + chunk - 1) / chunk;
  ProfScope prof(MOE_STAGE_CHUNK_COUNTS, s);
  hipError_t err = launch_fill_i32(chunk_counts, n_chunks * E, 0, s);
  if (err != hipSuccess || T <= 0) return err;
  const int64_t slots = T * k;
  chunk_hist_kernel<<<static_cast<unsigned>((slots + 255) / 256), 256, 0, s>>>(
      ids, slots, k, E, chunk, chunk_counts);
  return hipGetLastError();
}

}  // namespace moe
