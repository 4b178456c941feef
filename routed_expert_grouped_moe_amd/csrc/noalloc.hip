// moe_prefill_chunk_noalloc: the chunk call with a workspace the library holds itself, for
// callers that cannot allocate device memory.
//
// The workspace is a device array of this file's code object: each device the library runs
// on holds its own copy from the first call on that device until the process ends. In host
// code the array's name only stands in for it; its device address comes from
// hipGetSymbolAddress once per device (with that device current) and is kept per device, and
// only that address is handed to the kernels. Calls that overlap on one device share the
// array and race; the chunk's kernels write every workspace word they read (counts are cleared
// by a fill kernel), so nothing has to start at zero.
#include <mutex>
#include <unordered_map>

#include "moe_internal.h"
#include "ring.h"

namespace moe {
namespace {

constexpr size_t kScratchBytes = size_t{128} << 20;    // 128 MiB per device

static __device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_mu;
std::unordered_map<int, void*> g_scratch;               // device -> address of its array

void* scratch_of_device(moe_status* st) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) {
    *st = set_error(MOE_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(err));
    return nullptr;
  }
  std::lock_guard<std::mutex> lk(g_mu);
  auto it = g_scratch.find(dev);
  if (it != g_scratch.end()) return it->second;
  void* p = nullptr;
  err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (err != hipSuccess || !p) {
    *st = set_error(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                    hipGetErrorString(err));
    return nullptr;
  }
  g_scratch[dev] = p;
  return p;
}

}  // namespace
}  // namespace moe

extern "C" {

size_t moe_noalloc_workspace_bytes(void) { return moe::kScratchBytes; }

moe_status moe_prefill_chunk_noalloc(const moe_layer* layer, const void* x, const int32_t* ids,
                                     const float* weights, int64_t T, int64_t t0, int64_t n,
                                     void* out, void* stream) {
  moe::clear_error();
  return moe::prefill_chunk_checked(layer, x, ids, weights, T, t0, n, nullptr, out, nullptr,
                                    moe::kScratchBytes, stream, nullptr,
                                    /*resident_only=*/true, moe::scratch_of_device);
}

}  // extern "C"
