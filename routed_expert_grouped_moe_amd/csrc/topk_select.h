// Top-k selection by one wavefront, for one token or several whose reductions are interleaved.
#pragma once

#include <math.h>

#include "device_common.h"

namespace moe {

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

// One step of a wavefront maximum of 64-bit values (the two halves moved by DPP together).
template <int kCtrl, int kRowMask>
__device__ __forceinline__ uint64_t dpp_max64_step(uint64_t m) {
  const int lo = static_cast<int>(static_cast<uint32_t>(m));
  const int hi = static_cast<int>(static_cast<uint32_t>(m >> 32));
  const uint64_t o =
      (static_cast<uint64_t>(static_cast<uint32_t>(
           __builtin_amdgcn_update_dpp(hi, hi, kCtrl, kRowMask, 0xF, false))) << 32) |
      static_cast<uint32_t>(__builtin_amdgcn_update_dpp(lo, lo, kCtrl, kRowMask, 0xF, false));
  return o > m ? o : m;
}
// Wavefront maxima of NT independent values, their DPP steps interleaved: within quads
// (quad_perm [1,0,3,2] and [2,3,0,1]), mirrored half rows and rows, then the row broadcasts 15
// (into rows 1 and 3) and 31 (into rows 2 and 3). The result, valid in lane 63, is returned
// uniform.
template <int NT>
__device__ __forceinline__ void wave_max64(uint64_t (&m)[NT]) {
#pragma unroll
  for (int u = 0; u < NT; ++u) m[u] = dpp_max64_step<0xB1, 0xF>(m[u]);
#pragma unroll
  for (int u = 0; u < NT; ++u) m[u] = dpp_max64_step<0x4E, 0xF>(m[u]);
#pragma unroll
  for (int u = 0; u < NT; ++u) m[u] = dpp_max64_step<0x141, 0xF>(m[u]);
#pragma unroll
  for (int u = 0; u < NT; ++u) m[u] = dpp_max64_step<0x140, 0xF>(m[u]);
#pragma unroll
  for (int u = 0; u < NT; ++u) m[u] = dpp_max64_step<0x142, 0xA>(m[u]);
#pragma unroll
  for (int u = 0; u < NT; ++u) m[u] = dpp_max64_step<0x143, 0xC>(m[u]);
#pragma unroll
  for (int u = 0; u < NT; ++u) {
    const uint32_t lo = static_cast<uint32_t>(
        __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(m[u])), 63));
    const uint32_t hi = static_cast<uint32_t>(
        __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(m[u] >> 32)), 63));
    m[u] = (static_cast<uint64_t>(hi) << 32) | lo;
  }
}

// Top-k of NT tokens at once, one wavefront. For token u, lane l holds x[u][j] = the logit of
// expert l + 64 j (j < NJ; experts >= E are ignored). k rounds pick the k largest logits, the
// lower id among equal values, NaN ranking as -inf (and -0 as +0): a round takes, per token,
// the wavefront maximum of (key, ~id) over the untaken entries -- the largest key and, among
// equal keys, the lowest id -- and clears that entry. The chosen ids are written in ascending
// order by a ballot compaction, and each weight is
// exp(l - l_max) / (sum over the chosen of exp(l' - l_max), taken in ascending id), which
// equals the softmax over all experts renormalised over the chosen ones. The NT tokens'
// reductions are interleaved so their latencies overlap.
// ex[u]: LDS scratch of at least k floats for token u, used by this wavefront only. Writes
// ids_row[u][0..k) and w_row[u][0..k) of each active token. Every lane of the wavefront must
// call it.
template <int NJ, int NT>
__device__ __forceinline__ void topk_select(const float (&x)[NT][NJ], int E, int k,
                                            const bool (&active)[NT],
                                            int32_t* const (&ids_row)[NT],
                                            float* const (&w_row)[NT], float* const (&ex)[NT]) {
  const int lane = threadIdx.x & 63;
  float v[NT][NJ];
  uint32_t key[NT][NJ];
#pragma unroll
  for (int u = 0; u < NT; ++u)
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int e = lane + 64 * j;
      float xv = e < E ? x[u][j] : -INFINITY;
      if (xv != xv) xv = -INFINITY;
      if (xv == 0.f) xv = 0.f;     // -0 and +0 are equal logits: one key for both
      v[u][j] = xv;
      key[u][j] = e < E ? order_key(xv) : 0u;
    }
  uint32_t taken[NT];
  float vmax[NT];
#pragma unroll
  for (int u = 0; u < NT; ++u) {
    taken[u] = 0;
    vmax[u] = 0.f;
  }
  for (int r = 0; r < k; ++r) {
    uint64_t best[NT];
#pragma unroll
    for (int u = 0; u < NT; ++u) {
      uint32_t m = key[u][0];
      int jm = 0;
#pragma unroll
      for (int j = 1; j < NJ; ++j)    // strict: the lowest slice among equal keys
        if (key[u][j] > m) {
          m = key[u][j];
          jm = j;
        }
      best[u] = (static_cast<uint64_t>(m) << 32) |
                static_cast<uint32_t>(~static_cast<uint32_t>(lane + 64 * jm));
    }
    wave_max64<NT>(best);
#pragma unroll
    for (int u = 0; u < NT; ++u) {
      const uint32_t id = ~static_cast<uint32_t>(best[u]);
      const int lw = static_cast<int>(id & 63u), jw = static_cast<int>(id >> 6);
      if (r == 0) vmax[u] = key_value(static_cast<uint32_t>(best[u] >> 32));
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        if (lane == lw && j == jw) {
          key[u][j] = 0u;
          taken[u] |= 1u << j;
        }
    }
  }
#pragma unroll
  for (int u = 0; u < NT; ++u) {
    float* exu = ex[u];
    int base = 0;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const bool tk = (taken[u] >> j) & 1u;
      const uint64_t m = __ballot(tk);
      if (tk) {
        const int pos = base + __popcll(m & ((1ull << lane) - 1ull));
        if (active[u]) ids_row[u][pos] = lane + 64 * j;
        exu[pos] = v[u][j];
      }
      base += __popcll(m);
    }
  }
  // ex is this wavefront's own: its LDS operations complete in order
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int u = 0; u < NT; ++u)
    for (int p = lane; p < k; p += 64) ex[u][p] = expf(ex[u][p] - vmax[u]);
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int u = 0; u < NT; ++u) {
    float sum = 0.f;
    if (lane == 0)
      for (int p = 0; p < k; ++p) sum += ex[u][p];
    sum = __shfl(sum, 0);
    if (active[u])
      for (int p = lane; p < k; p += 64) w_row[u][p] = ex[u][p] / sum;
  }
  __builtin_amdgcn_wave_barrier();
}

}  // namespace moe
