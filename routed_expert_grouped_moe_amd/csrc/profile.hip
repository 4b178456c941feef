// Opt-in per-stage kernel timing with HIP events recorded on each launch's own stream.
#include <mutex>
#include <unordered_map>
#include <vector>

#include "profile.h"
#include "ring.h"

namespace moe {
namespace {

struct Pending {
  int stage;
  hipEvent_t a, b;
};

std::mutex g_mu;
bool g_on = false;
std::vector<Pending> g_pending;
std::vector<hipEvent_t> g_pool;
double g_ms[MOE_PROFILE_SLOTS];
int64_t g_n[MOE_PROFILE_SLOTS];
double g_clk[MOE_PROFILE_SLOTS], g_rt[MOE_PROFILE_SLOTS];                        // summed clock samples read back so far
std::unordered_map<int, unsigned long long*> g_clk_dev;   // per device: [slots][2] counters

// The clock counters live in a device array of the library's own code object (each device
// holds its own copy), so profiling allocates no device memory. In host code the array's name
// is only a stand-in: its device address comes from hipGetSymbolAddress, once per device.
__device__ __align__(256) unsigned long long g_clk_counters[MOE_PROFILE_SLOTS * 2];

static_assert(MOE_STAGE_COUNT <= MOE_PROFILE_SLOTS, "a profile slot per stage");

hipEvent_t take_event() {   // caller holds g_mu
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

unsigned long long* prof_clock(int stage) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_on || stage < 0 || stage >= MOE_PROFILE_SLOTS) return nullptr;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  unsigned long long*& buf = g_clk_dev[dev];
  if (!buf) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(g_clk_counters)) != hipSuccess || !p) return nullptr;
    if (hipMemset(p, 0, MOE_PROFILE_SLOTS * 2 * sizeof(unsigned long long)) != hipSuccess) return nullptr;
    buf = static_cast<unsigned long long*>(p);
  }
  return buf + 2 * stage;
}

ProfScope::ProfScope(int stage, hipStream_t s) : stage_(stage), s_(s) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_on) return;
  a_ = take_event();
  if (a_ && hipEventRecord(a_, s_) != hipSuccess) {
    g_pool.push_back(a_);
    a_ = nullptr;
  }
}

ProfScope::~ProfScope() {
  if (!a_) return;
  std::lock_guard<std::mutex> lk(g_mu);
  hipEvent_t b = take_event();
  if (b && hipEventRecord(b, s_) == hipSuccess) {
    g_pending.push_back({stage_, a_, b});
  } else {
    g_pool.push_back(a_);
    if (b) g_pool.push_back(b);
  }
}

}  // namespace moe

extern "C" {

moe_status moe_profile_enable(int32_t on) {
  std::lock_guard<std::mutex> lk(moe::g_mu);
  moe::g_on = on != 0;
  return MOE_OK;
}

moe_status moe_profile_read(moe_profile_t* out, int32_t reset) {
  moe::clear_error();
  if (!out) return moe::set_error(MOE_ERR_INVALID, "out is NULL");
  std::lock_guard<std::mutex> lk(moe::g_mu);
  moe_status st = MOE_OK;
  for (const moe::Pending& p : moe::g_pending) {
    float ms = 0.f;
    hipError_t err = hipEventSynchronize(p.b);
    if (err == hipSuccess) err = hipEventElapsedTime(&ms, p.a, p.b);
    if (err != hipSuccess && st == MOE_OK)
      st = moe::set_error(MOE_ERR_HIP, "profile events: %s", hipGetErrorString(err));
    moe::g_ms[p.stage] += ms;
    moe::g_n[p.stage] += 1;
    moe::g_pool.push_back(p.a);
    moe::g_pool.push_back(p.b);
  }
  moe::g_pending.clear();
  for (auto& kv : moe::g_clk_dev) {              // every launch read above has completed
    if (!kv.second) continue;
    unsigned long long h[MOE_PROFILE_SLOTS * 2];
    int cur = 0;
    hipError_t err = hipGetDevice(&cur);
    if (err == hipSuccess) err = hipSetDevice(kv.first);
    if (err == hipSuccess) err = hipMemcpy(h, kv.second, sizeof(h), hipMemcpyDeviceToHost);
    if (err == hipSuccess) err = hipMemset(kv.second, 0, sizeof(h));
    (void)hipSetDevice(cur);
    if (err != hipSuccess) {
      if (st == MOE_OK) st = moe::set_error(MOE_ERR_HIP, "profile clocks: %s", hipGetErrorString(err));
      continue;
    }
    for (int i = 0; i < MOE_PROFILE_SLOTS; ++i) {
      moe::g_clk[i] += static_cast<double>(h[2 * i]);
      moe::g_rt[i] += static_cast<double>(h[2 * i + 1]);
    }
  }
  out->version = 3;
  out->n_stages = MOE_STAGE_COUNT;
  for (int i = 0; i < MOE_PROFILE_SLOTS; ++i) {
    out->ms[i] = moe::g_ms[i];
    out->launches[i] = moe::g_n[i];
    out->clock_mhz[i] = moe::g_rt[i] > 0 ? moe::g_clk[i] / moe::g_rt[i] * 100.0 : 0.0;
    if (reset) {
      moe::g_ms[i] = 0.0;
      moe::g_n[i] = 0;
      moe::g_clk[i] = 0.0;
      moe::g_rt[i] = 0.0;
    }
  }
  return st;
}

}  // extern "C"
