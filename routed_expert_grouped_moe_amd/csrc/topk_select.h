// Top-k selection of one token by one wavefront.
#pragma once

#include <math.h>

#include "device_common.h"

namespace moe {

// Orderable 32-bit key of a float: a > b as floats (no NaN) iff key(a) > key(b) as unsigned.
// Every key of a real value is at least 0x007FFFFF (the key of -inf), so 0 can mark a missing
// entry.
__device__ __forceinline__ uint32_t order_key(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

// One step of a wavefront maximum of 32-bit unsigned values by DPP. A lane whose source row
// is masked off reads 0, the identity of the maximum.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ uint32_t dpp_max32_step(uint32_t m) {
  const uint32_t o = static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(m), kCtrl, kRowMask, 0xF, false));
  return o > m ? o : m;
}
// Wavefront maximum: within quads (quad_perm [1,0,3,2] and [2,3,0,1]), mirrored half rows and
// rows, then the row broadcasts 15 (into rows 1 and 3) and 31 (into rows 2 and 3). The result,
// valid in lane 63, is returned uniform.
__device__ __forceinline__ uint32_t wave_max32(uint32_t m) {
  m = dpp_max32_step<0xB1, 0xF>(m);
  m = dpp_max32_step<0x4E, 0xF>(m);
  m = dpp_max32_step<0x141, 0xF>(m);
  m = dpp_max32_step<0x140, 0xF>(m);
  m = dpp_max32_step<0x142, 0xA>(m);
  m = dpp_max32_step<0x143, 0xC>(m);
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(m), 63));
}

// Sorts a lane's N values (a power of two) into descending order: a bitonic network, every
// compare-exchange on fixed registers.
template <int N>
__device__ __forceinline__ void sort_desc(uint64_t (&a)[N]) {
#pragma unroll
  for (int size = 2; size <= N; size <<= 1)
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1)
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const int l = i ^ stride;
        if (l > i) {
          const bool down = (i & size) == 0;     // this pair ends in descending order
          const bool lt = a[i] < a[l];
          const uint64_t lo = lt ? a[i] : a[l], hi = lt ? a[l] : a[i];
          a[i] = down ? hi : lo;
          a[l] = down ? lo : hi;
        }
      }
}

// LDS words (8 bytes) topk_select needs per token: each lane's sorted list plus a zero.
template <int NJ>
constexpr int topk_lds_words() { return 64 * (NJ + 1); }

// Top-k of one token by one wavefront. Lane l holds x[j] = the logit of expert l * NJ + j
// (j < NJ, NJ a power of two; experts >= E are ignored). The k largest logits are picked, the
// lower id among equal values, NaN ranking as -inf (and -0 as +0):
//  * each lane sorts its entries once by (key, NJ - 1 - j) descending, so its list runs in
//    the order the selection takes them, and keeps it in LDS;
//  * a round takes the wavefront maximum of the lanes' first untaken keys; among the lanes
//    holding it the lowest lane has the lowest id (lane l holds ids l*NJ .. l*NJ + NJ - 1),
//    and its first untaken entry is its lowest id with that key; that lane moves one entry on.
// The chosen ids are written in ascending order (lane by lane, ascending j within a lane),
// and each weight is exp(l - l_max) / (sum over the chosen of exp(l' - l_max), taken in
// ascending id), which equals the softmax over all experts renormalised over the chosen ones.
// lst: LDS of topk_lds_words<NJ>() words for this wavefront only (it also holds the k
// exponentials afterwards). Writes ids_row[0..k) and w_row[0..k) if `active`. Every lane of
// the wavefront must call it.
template <int NJ>
__device__ __forceinline__ void topk_select(const float (&x)[NJ], int E, int k, bool active,
                                            int32_t* ids_row, float* w_row, uint64_t* lst) {
  const int lane = threadIdx.x & 63;
  float v[NJ];
  uint64_t c[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int e = lane * NJ + j;
    float xv = e < E ? x[j] : -INFINITY;
    if (xv != xv) xv = -INFINITY;
    if (xv == 0.f) xv = 0.f;     // -0 and +0 are equal logits: one key for both
    v[j] = xv;
    // every key of a real value is above 0 (the key of -inf is 0x007FFFFF): 0 marks "none"
    c[j] = e < E ? (static_cast<uint64_t>(order_key(xv)) << 32) | static_cast<uint32_t>(NJ - 1 - j)
                 : 0ull;
  }
  sort_desc<NJ>(c);
#pragma unroll
  for (int s = 0; s < NJ; ++s) lst[s * 64 + lane] = c[s];
  lst[NJ * 64 + lane] = 0ull;
  uint64_t head = c[0];
  int p = 0;                    // entries this lane has given up
  float vmax = 0.f;
  for (int r = 0; r < k; ++r) {
    // k <= E, so an untaken real entry (key above 0) is left in every round
    const uint32_t hk = static_cast<uint32_t>(head >> 32);
    const uint32_t km = wave_max32(hk);
    if (r == 0) vmax = key_value(km);
    const uint64_t b = __ballot(hk == km);
    if (lane == __ffsll(static_cast<long long>(b)) - 1) {
      ++p;
      head = lst[p * 64 + lane];
    }
  }
  uint32_t mask = 0;            // j of the lane's chosen entries
#pragma unroll
  for (int s = 0; s < NJ; ++s)
    if (s < p) mask |= 1u << (NJ - 1 - static_cast<int>(static_cast<uint32_t>(c[s])));
  const int cnt = __popc(mask);
  int base = 0;                 // chosen entries of the lanes below
  for (int q = 1; q <= NJ; ++q) {
    const uint64_t m = __ballot(cnt >= q);
    if (!m) break;
    base += __popcll(m & ((1ull << lane) - 1ull));
  }
  // lst is this wavefront's own and its LDS operations complete in order: the list reads above
  // are done before these writes reuse the space
  float* ex = reinterpret_cast<float*>(lst);
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int j = 0, pos = base; j < NJ; ++j)
    if ((mask >> j) & 1u) {
      if (active) ids_row[pos] = lane * NJ + j;
      ex[pos] = v[j];
      ++pos;
    }
  __builtin_amdgcn_wave_barrier();
  for (int q = lane; q < k; q += 64) ex[q] = expf(ex[q] - vmax);
  __builtin_amdgcn_wave_barrier();
  float sum = 0.f;
  if (lane == 0)
    for (int q = 0; q < k; ++q) sum += ex[q];
  sum = __shfl(sum, 0);
  if (active)
    for (int q = lane; q < k; q += 64) w_row[q] = ex[q] / sum;
  __builtin_amdgcn_wave_barrier();
}

}  // namespace moe
