// Copy of one expert line from a pinned host bank into a ring line, as a kernel.
//
// The ring's copies wait on release events recorded on the compute stream after the GEMMs that
// read the lines. A DMA-engine copy behind such a wait leaves the link idle for a while each
// time (measured on the box: 6 MiB copies on two streams move 57 GB/s alone, 30-56 GB/s with one
// such wait per 16 copies), while a kernel reading the pinned bank through its device mapping
// keeps 54.5-55 GB/s with the same waits, from 16 workgroups: a stream-to-stream dependency
// between two kernels costs next to nothing. Each workgroup copies a contiguous share of the
// line in 16-byte vectors, 4 in flight per thread, with non-temporal loads (the bank is read
// once) and plain stores (the GEMMs read the line next).
#include "device_common.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kCopyBlocks = 16, kCopyThreads = 256, kCopyUnroll = 4;

__global__ __launch_bounds__(kCopyThreads) void line_copy_kernel(const u32x4_t* __restrict__ src,
                                                                  u32x4_t* __restrict__ dst,
                                                                  int64_t n16) {
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t lo = static_cast<int64_t>(blockIdx.x) * per;
  const int64_t hi = lo + per < n16 ? lo + per : n16;
  for (int64_t i = lo + threadIdx.x; i < hi; i += kCopyThreads * kCopyUnroll) {
    u32x4_t v[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const int64_t j = i + static_cast<int64_t>(u) * kCopyThreads;
      v[u] = j < hi ? __builtin_nontemporal_load(src + j) : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const int64_t j = i + static_cast<int64_t>(u) * kCopyThreads;
      if (j < hi) dst[j] = v[u];
    }
  }
}

}  // namespace

hipError_t launch_line_copy(void* dst, const void* src_dev, size_t bytes, hipStream_t s) {
  if (bytes == 0) return hipSuccess;
  line_copy_kernel<<<kCopyBlocks, kCopyThreads, 0, s>>>(
      static_cast<const u32x4_t*>(src_dev), static_cast<u32x4_t*>(dst),
      static_cast<int64_t>(bytes / 16));
  return hipGetLastError();
}

}  // namespace moe
