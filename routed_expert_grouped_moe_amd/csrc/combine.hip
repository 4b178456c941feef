// The combine (one fixed reduction order per token) and the RMSNorm + residual glue of a stack.
#include <math.h>

#include "device_common.h"
#include "moe_internal.h"
#include "profile.h"

namespace moe {
namespace {

template <typename T> struct Pack4;
template <> struct Pack4<uint16_t> {
  static __device__ __forceinline__ void store(uint16_t* p, float4 v) {
    uint2 w;
    w.x = f32x2_to_bf16x2(v.x, v.y);
    w.y = f32x2_to_bf16x2(v.z, v.w);
    *reinterpret_cast<uint2*>(p) = w;
  }
  static __device__ __forceinline__ float4 load(const uint16_t* p) {
    const uint2 w = *reinterpret_cast<const uint2*>(p);
    return make_float4(bf16_to_f32(w.x & 0xffffu), bf16_to_f32(w.x >> 16),
                       bf16_to_f32(w.y & 0xffffu), bf16_to_f32(w.y >> 16));
  }
};
template <> struct Pack4<float> {
  static __device__ __forceinline__ void store(float* p, float4 v) {
    *reinterpret_cast<float4*>(p) = v;
  }
  static __device__ __forceinline__ float4 load(const float* p) {
    return *reinterpret_cast<const float4*>(p);
  }
};

// The canonical reduction of one token (the routed-expert reduction the exact deep prefill
// page, "Flash Next EXL3: exact deep prefill", adopts so chunk size cannot change a sum):
//   acc = 0; for each chosen expert in ascending id: acc = fma(w_j, y_j, acc); acc += shared;
//   out = round(acc)    (one rounding to the storage type, bf16 round-to-nearest-even)
// y_j is the unweighted fp32 row expert j wrote for this token; the order never depends on
// the chunk, the expert's row count or where the expert ran.
//
// Y is read once: non-temporal loads keep it from displacing cached data.
__device__ __forceinline__ float4 load_stream(const float* p) {
  const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
  return make_float4(v[0], v[1], v[2], v[3]);
}

// A thread owns 4-column groups c and c + 1024 (d = 2048 is one pass) and issues the loads of
// 8 expert rows before their FMAs, which run in the same ascending order.
template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y,
                                                      const float* __restrict__ shared,
                                                      const float* __restrict__ weights,
                                                      int64_t t0, int k, int d,
                                                      T* __restrict__ out) {
  constexpr int U = 2, J = 8;
  const int64_t t = blockIdx.x;                       // token within the chunk
  const float* wt = weights + (t0 + t) * k;
  const float* yt = y + t * k * static_cast<int64_t>(d);
  for (int c0 = threadIdx.x * 4; c0 < d; c0 += 1024 * U) {
    float4 acc[U];
    bool on[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      acc[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      on[u] = c0 + 1024 * u < d;
    }
    int j = 0;
    for (; j + J <= k; j += J) {
      float4 v[J][U];
#pragma unroll
      for (int i = 0; i < J; ++i)
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (on[u])
            v[i][u] = load_stream(yt + static_cast<int64_t>(MOE_SLOT(j + i, k)) * d + c0 + 1024 * u);
#pragma unroll
      for (int i = 0; i < J; ++i) {
        const float wj = wt[MOE_SLOT(j + i, k)];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          acc[u].x = fmaf(wj, v[i][u].x, acc[u].x);
          acc[u].y = fmaf(wj, v[i][u].y, acc[u].y);
          acc[u].z = fmaf(wj, v[i][u].z, acc[u].z);
          acc[u].w = fmaf(wj, v[i][u].w, acc[u].w);
        }
      }
    }
    for (; j < k; ++j) {
      const float wj = wt[MOE_SLOT(j, k)];
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (on[u]) {
          const float4 v = load_stream(yt + static_cast<int64_t>(MOE_SLOT(j, k)) * d + c0 + 1024 * u);
          acc[u].x = fmaf(wj, v.x, acc[u].x);
          acc[u].y = fmaf(wj, v.y, acc[u].y);
          acc[u].z = fmaf(wj, v.z, acc[u].z);
          acc[u].w = fmaf(wj, v.w, acc[u].w);
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (!on[u]) continue;
      const int c = c0 + 1024 * u;
      if (shared) {
        const float4 s = *reinterpret_cast<const float4*>(shared + t * d + c);
        acc[u].x = routed_sum<T>(acc[u].x) + s.x;
        acc[u].y = routed_sum<T>(acc[u].y) + s.y;
        acc[u].z = routed_sum<T>(acc[u].z) + s.z;
        acc[u].w = routed_sum<T>(acc[u].w) + s.w;
      }
      Pack4<T>::store(out + (t0 + t) * d + c, acc[u]);
    }
  }
}

// x_new = round(x + delta) (when delta is given); normed = round(x_new / sqrt(mean(x_new^2) +
// eps)). x_out may be x itself (each element is read before the same thread overwrites it), so
// neither carries __restrict__. Each thread sums squares of columns tid, tid + 256, ... in order, then a fixed
// halving tree over the 256 partial sums: the same bits on every run.
template <typename T>
__global__ __launch_bounds__(256) void add_rmsnorm_kernel(const T* x,
                                                          const T* __restrict__ delta, int d,
                                                          float eps, T* x_out,
                                                          T* __restrict__ normed) {
  __shared__ float red[256];
  const int tid = threadIdx.x;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * d;
  float ss = 0.f;
  for (int c = tid; c < d; c += 256) {
    float v = Elt<T>::load(x[row + c]);
    if (delta) {
      const T r = Elt<T>::store(v + Elt<T>::load(delta[row + c]));
      x_out[row + c] = r;
      v = Elt<T>::load(r);
    }
    ss = fmaf(v, v, ss);
  }
  red[tid] = ss;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) red[tid] += red[tid + s];
    __syncthreads();
  }
  const float inv = 1.0f / sqrtf(red[0] / static_cast<float>(d) + eps);
  for (int c = tid; c < d; c += 256) {
    const float v = Elt<T>::load(delta ? x_out[row + c] : x[row + c]);
    normed[row + c] = Elt<T>::store(v * inv);
  }
}

}  // namespace

hipError_t launch_combine(int dtype, const float* y, const float* shared, const float* weights,
                          int64_t t0, int64_t n, int k, int d, void* out, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  ProfScope prof(MOE_STAGE_COMBINE, s);
  if (dtype == MOE_BF16)
    combine_kernel<uint16_t><<<static_cast<unsigned>(n), 256, 0, s>>>(
        y, shared, weights, t0, k, d, static_cast<uint16_t*>(out));
  else
    combine_kernel<float><<<static_cast<unsigned>(n), 256, 0, s>>>(
        y, shared, weights, t0, k, d, static_cast<float*>(out));
  return hipGetLastError();
}

hipError_t launch_add_rmsnorm(int dtype, const void* x, const void* delta, int64_t T, int d,
                              float eps, void* x_out, void* normed, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  ProfScope prof(MOE_STAGE_RMSNORM, s);
  if (dtype == MOE_BF16)
    add_rmsnorm_kernel<uint16_t><<<static_cast<unsigned>(T), 256, 0, s>>>(
        static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(delta), d, eps,
        static_cast<uint16_t*>(x_out), static_cast<uint16_t*>(normed));
  else
    add_rmsnorm_kernel<float><<<static_cast<unsigned>(T), 256, 0, s>>>(
        static_cast<const float*>(x), static_cast<const float*>(delta), d, eps,
        static_cast<float*>(x_out), static_cast<float*>(normed));
  return hipGetLastError();
}

}  // namespace moe
