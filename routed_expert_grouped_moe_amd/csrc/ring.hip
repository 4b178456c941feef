// Ring of device expert lines fed from pinned host banks by asynchronous copies.
//
// The pages' design ("deep prefill (slice 3 of 7)", PR #1443, What; "EXL3 on upstream",
// PR #1113, Loading, "Latest prefill efficiency candidate" and "Latest measured follow-up"):
// routed experts live in pinned host banks and are staged into a pool of device lines by
// host-planned asynchronous host-to-device copies that overlap compute; lines keep experts
// for reuse; a copy into a line waits for the line's readers through release epochs, and
// waits on epochs already covered are coalesced; an expert whose projections are adjacent in
// the bank moves in one copy. Here every expert line is contiguous (W_gu then W_down), so a
// miss is exactly one hipMemcpyAsync on the copy stream, followed by the line's `ready` event.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <string>

#include "ring.h"

namespace moe {

namespace {
thread_local std::string g_last_error;
}  // namespace

moe_status set_error(moe_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

const char* last_error_text() { return g_last_error.c_str(); }
void clear_error() { g_last_error.clear(); }

moe_status ring_stage(moe_ring* r, int32_t layer, const int32_t* experts, int32_t n,
                      hipStream_t cs0, int32_t* lines_out, const std::vector<char>* later,
                      bool two_streams, int kind, bool hold, bool kernel_copy) {
  if (kind < 0 || kind >= MOE_COPY_KINDS) kind = MOE_COPY_DEMAND;
  auto bit = r->banks.find(layer);
  if (bit == r->banks.end())
    return set_error(MOE_ERR_RING, "no bank bound for layer %d", layer);
  const moe_ring::Bank& bank = bit->second;
  const int E = r->shape.n_experts;
  std::vector<char> seen(E, 0);
  std::vector<int32_t> hit_line(n, -1);
  int misses = 0;
  for (int i = 0; i < n; ++i) {
    const int e = experts[i];
    if (e < 0 || e >= E) return set_error(MOE_ERR_INVALID, "expert %d out of range", e);
    if (seen[e]) return set_error(MOE_ERR_INVALID, "expert %d listed twice", e);
    seen[e] = 1;
    if (bank.slot[e] < 0)
      return set_error(MOE_ERR_INVALID, "expert %d of layer %d is not in the bank", e, layer);
    auto w = r->where.find(ring_key(layer, e));
    if (w != r->where.end()) hit_line[i] = w->second;
    else ++misses;
  }
  int free_lines = 0;
  {
    std::vector<char> taken(r->n_lines, 0);
    for (int i = 0; i < n; ++i)
      if (hit_line[i] >= 0) taken[hit_line[i]] = 1;
    for (int l = 0; l < r->n_lines; ++l)
      if (!r->line[l].held && !taken[l]) ++free_lines;
  }
  if (misses > free_lines)
    return set_error(MOE_ERR_RING, "%d experts to copy but only %d lines free", misses,
                     free_lines);

  if (two_streams && misses > 1 && !r->copy2) {
    hipError_t err = hipStreamCreateWithFlags(&r->copy2, hipStreamNonBlocking);
    if (err != hipSuccess) {
      r->copy2 = nullptr;
      return set_error(MOE_ERR_HIP, "hipStreamCreateWithFlags: %s", hipGetErrorString(err));
    }
  }
  const bool split = two_streams && r->copy2 != nullptr;
  int miss_no = 0;
  for (int i = 0; i < n; ++i) {            // hits first: they must not be chosen as victims
    if (hit_line[i] < 0) continue;
    moe_ring::Line& ln = r->line[hit_line[i]];
    if (hold) ln.held = true;
    ln.last_use = ++r->clock;
    r->stats.hits++;
    r->stats.requested_bytes[kind] += static_cast<int64_t>(r->line_bytes);
    if (lines_out) lines_out[i] = hit_line[i];
  }
  // Misses in three passes: choose every victim, then make each copy stream wait once per
  // release stream for the newest release among its victims (releases recorded on one stream
  // complete in order, so that wait covers the older ones), then issue the copies.
  struct Planned {
    int i, victim, sj;
  };
  std::vector<Planned> plan;
  plan.reserve(misses);
  for (int i = 0; i < n; ++i) {
    if (hit_line[i] >= 0) continue;
    int victim = -1, victim_needed = -1;
    for (int l = 0; l < r->n_lines; ++l) {
      const moe_ring::Line& c = r->line[l];
      if (c.held) continue;
      const bool needed = later && c.layer == layer && c.expert >= 0 && (*later)[c.expert];
      int& v = needed ? victim_needed : victim;
      if (v < 0 || c.last_use < r->line[v].last_use) v = l;
    }
    if (victim < 0) victim = victim_needed;
    moe_ring::Line& ln = r->line[victim];
    if (ln.expert >= 0) r->where.erase(ring_key(ln.layer, ln.expert));
    ln.layer = -1;
    ln.expert = -1;
    ln.held = true;
    plan.push_back({i, victim, split ? (miss_no++ & 1) : 0});
  }
  // On a HIP error nothing this call took stays held: hit lines and filled victims keep their
  // (valid) contents, victims not yet filled stay empty.
  auto unwind = [&](size_t) {
    if (hold)
      for (int i = 0; i < n; ++i)
        if (hit_line[i] >= 0) r->line[hit_line[i]].held = false;
    for (const Planned& pl : plan) r->line[pl.victim].held = false;
  };
  for (int sj = 0; sj < 2; ++sj) {
    hipStream_t cs = sj ? r->copy2 : cs0;
    moe_ring::Coal& co = r->coal[sj];
    std::vector<int> newest;                 // per release stream: victim of the newest release
    for (const Planned& pl : plan) {
      if (pl.sj != sj || !r->line[pl.victim].has_release) continue;
      const moe_ring::Line& ln = r->line[pl.victim];
      bool merged = false;
      for (int& v : newest)
        if (r->line[v].release_stream == ln.release_stream) {
          if (ln.release_seq > r->line[v].release_seq) v = pl.victim;
          merged = true;
        }
      if (!merged) newest.push_back(pl.victim);
    }
    for (int v : newest) {
      const moe_ring::Line& ln = r->line[v];
      if (ln.release_stream == co.rel && cs == co.copy && ln.release_seq <= co.seq) continue;
      hipError_t err = hipStreamWaitEvent(cs, r->release[v], 0);
      if (err != hipSuccess) {
        unwind(0);
        return set_error(MOE_ERR_HIP, "hipStreamWaitEvent(release): %s", hipGetErrorString(err));
      }
      if (ln.release_stream != co.rel || cs != co.copy) {
        co.rel = ln.release_stream;
        co.copy = cs;
        co.seq = 0;
      }
      co.seq = std::max(co.seq, ln.release_seq);
      r->stats.copy_waits++;
    }
  }
  for (size_t q = 0; q < plan.size(); ++q) {
    const Planned& pl = plan[q];
    hipStream_t cs = pl.sj ? r->copy2 : cs0;
    const int e = experts[pl.i];
    const size_t src_off = static_cast<size_t>(bank.slot[e]) * r->line_bytes;
    char* dst = r->lines + static_cast<size_t>(pl.victim) * r->line_bytes;
    hipError_t err = (kernel_copy && bank.dev_base)
                         ? launch_line_copy(dst, bank.dev_base + src_off, r->line_bytes, cs)
                         : hipMemcpyAsync(dst, bank.base + src_off, r->line_bytes,
                                          hipMemcpyHostToDevice, cs);
    if (err == hipSuccess) err = hipEventRecord(r->ready[pl.victim], cs);
    // not held: the copy stream itself is the line's last reader so far
    if (err == hipSuccess && !hold) err = hipEventRecord(r->release[pl.victim], cs);
    if (err != hipSuccess) {
      unwind(q);
      return set_error(MOE_ERR_HIP, "copy into line %d: %s", pl.victim, hipGetErrorString(err));
    }
    moe_ring::Line& ln = r->line[pl.victim];
    ln.has_ready = true;
    ln.ready_seen_valid = false;           // a new fill: no stream has waited for it yet
    ln.layer = layer;
    ln.expert = e;
    ln.last_use = ++r->clock;
    if (!hold) {
      ln.held = false;
      ln.has_release = true;
      ln.release_seq = ++r->release_counter;
      ln.release_stream = cs;
      ln.ready_seen = cs;                  // the copy stream is ordered after its own copy
      ln.ready_seen_valid = true;
    }
    r->where[ring_key(layer, e)] = pl.victim;
    r->stats.misses++;
    r->stats.bytes_h2d += static_cast<int64_t>(r->line_bytes);
    r->stats.requested_bytes[kind] += static_cast<int64_t>(r->line_bytes);
    r->stats.copied_bytes[kind] += static_cast<int64_t>(r->line_bytes);
    if (lines_out) lines_out[pl.i] = pl.victim;
  }
  return MOE_OK;
}

moe_status ring_wait_ready(moe_ring* r, const int32_t* lines, int32_t n, hipStream_t s) {
  for (int i = 0; i < n; ++i) {
    const int l = lines[i];
    if (l < 0 || l >= r->n_lines) return set_error(MOE_ERR_INVALID, "line %d out of range", l);
    if (!r->line[l].has_ready) continue;
    hipError_t err = hipStreamWaitEvent(s, r->ready[l], 0);
    if (err != hipSuccess)
      return set_error(MOE_ERR_HIP, "hipStreamWaitEvent(ready): %s", hipGetErrorString(err));
    r->line[l].ready_seen = s;
    r->line[l].ready_seen_valid = true;
  }
  return MOE_OK;
}

moe_status ring_release(moe_ring* r, const int32_t* lines, int32_t n, hipStream_t s) {
  for (int i = 0; i < n; ++i) {
    const int l = lines[i];
    if (l < 0 || l >= r->n_lines) return set_error(MOE_ERR_INVALID, "line %d out of range", l);
    moe_ring::Line& ln = r->line[l];
    // The line's last release may be on another stream (an earlier reader released it there,
    // then a staging found it as a hit and handed it to this stream): the one release event
    // must cover both readers, so this stream first waits for the earlier release.
    hipError_t err = hipSuccess;
#if !defined(MOE_PLANT_RELEASE_ONE_STREAM)   // test-only build of the host check: no such wait
    if (ln.has_release && ln.release_stream != s) err = hipStreamWaitEvent(s, r->release[l], 0);
#endif
    // A holder that never waited for the line's fill on this stream (a staging released
    // without moe_ring_wait_ready) must not release it before the fill lands: a later copy
    // into the line waits only for the release.
#if !defined(MOE_PLANT_RELEASE_BEFORE_FILL)  // test-only build of the host check: no such wait
    if (err == hipSuccess && ln.has_ready && !(ln.ready_seen_valid && ln.ready_seen == s)) {
      err = hipStreamWaitEvent(s, r->ready[l], 0);
      ln.ready_seen = s;
      ln.ready_seen_valid = true;
    }
#endif
    if (err == hipSuccess) err = hipEventRecord(r->release[l], s);
    if (err != hipSuccess)
      return set_error(MOE_ERR_HIP, "release of line %d: %s", l, hipGetErrorString(err));
    ln.has_release = true;
    ln.release_seq = ++r->release_counter;
    ln.release_stream = s;
    ln.held = false;
  }
  return MOE_OK;
}

}  // namespace moe

using moe::set_error;

extern "C" {

moe_status moe_ring_create(const moe_shape* shape, void* device_lines, int32_t n_lines,
                           moe_ring** out) {
  moe::clear_error();
  if (!out) return set_error(MOE_ERR_INVALID, "out is NULL");
  *out = nullptr;
  if (!shape) return set_error(MOE_ERR_INVALID, "shape is NULL");
  if (!device_lines || (reinterpret_cast<uintptr_t>(device_lines) & 255u))
    return set_error(MOE_ERR_INVALID, "device_lines NULL or not 256-byte aligned");
  if (n_lines < 1 || n_lines > (1 << 20)) return set_error(MOE_ERR_INVALID, "n_lines %d", n_lines);
  if (moe_workspace_bytes(shape, 1) == 0) return set_error(MOE_ERR_INVALID, "invalid shape");
  moe_ring* r = new moe_ring();
  r->shape = *shape;
  const size_t elt = shape->dtype == MOE_BF16 ? 2 : 4;
  r->line_bytes = 3ull * shape->inter * shape->d * elt;
  r->lines = static_cast<char*>(device_lines);
  r->n_lines = n_lines;
  r->line.resize(n_lines);
  // test-only fault injection: make the N-th event creation fail (0 = off)
  int fail_at = 0;
  if (const char* f = getenv("MOE_TEST_FAIL_EVENT_CREATE")) fail_at = atoi(f);
  int made = 0;
  auto make = [&](hipEvent_t* ev) -> hipError_t {
    ++made;
    if (fail_at > 0 && made == fail_at) return hipErrorOutOfMemory;
    return hipEventCreateWithFlags(ev, hipEventDisableTiming);
  };
  hipError_t err = hipSuccess;
  for (int l = 0; l < n_lines && err == hipSuccess; ++l) {
    hipEvent_t a = nullptr, b = nullptr;
    err = make(&a);
    if (err == hipSuccess) r->ready.push_back(a);
    if (err == hipSuccess) {
      err = make(&b);
      if (err == hipSuccess) r->release.push_back(b);
    }
  }
  if (err != hipSuccess) {            // unwind: nothing stays allocated
    for (hipEvent_t e : r->ready) (void)hipEventDestroy(e);
    for (hipEvent_t e : r->release) (void)hipEventDestroy(e);
    delete r;
    return set_error(MOE_ERR_HIP, "hipEventCreateWithFlags: %s", hipGetErrorString(err));
  }
  r->stats.version = 3;
  r->stats.n_lines = n_lines;
  *out = r;
  return MOE_OK;
}

moe_status moe_ring_bind_bank(moe_ring* r, int32_t layer_id, const void* pinned_bank,
                              const int32_t* bank_slot_of_expert) {
  moe::clear_error();
  if (!r || layer_id < 0 || !bank_slot_of_expert)
    return set_error(MOE_ERR_INVALID, "bad ring, layer id or slot array");
  const int E = r->shape.n_experts;
  bool any = false;
  for (int e = 0; e < E; ++e) {
    if (bank_slot_of_expert[e] < -1) return set_error(MOE_ERR_INVALID, "slot of expert %d", e);
    any |= bank_slot_of_expert[e] >= 0;
  }
  if (any && !pinned_bank) return set_error(MOE_ERR_INVALID, "pinned_bank is NULL");
  for (auto it = r->where.begin(); it != r->where.end();) {   // drop the layer's cached lines
    if ((it->first >> 32) == layer_id) {
      moe_ring::Line& ln = r->line[it->second];
      ln.layer = -1;
      ln.expert = -1;
      ln.last_use = 0;
      it = r->where.erase(it);
    } else {
      ++it;
    }
  }
  moe_ring::Bank& b = r->banks[layer_id];
  b.base = static_cast<const char*>(pinned_bank);
  b.dev_base = nullptr;
  // The copy kernel reads the bank through the device's mapping of the pinned memory; it is
  // used only where that mapping is the host address itself (unified addressing) and 16-byte
  // aligned, else the copies stay with hipMemcpyAsync.
  if (pinned_bank) {
    void* dev = nullptr;
    if (hipHostGetDevicePointer(&dev, const_cast<void*>(pinned_bank), 0) == hipSuccess &&
        dev == pinned_bank && (reinterpret_cast<uintptr_t>(dev) & 15u) == 0 &&
        (r->line_bytes & 15u) == 0)
      b.dev_base = static_cast<const char*>(dev);
    else
      (void)hipGetLastError();        // leave no error behind for the next launch check
  }
  b.slot.assign(bank_slot_of_expert, bank_slot_of_expert + E);
  return MOE_OK;
}

moe_status moe_stage_experts(moe_ring* r, int32_t layer_id, const int32_t* experts, int32_t n,
                             void* copy_stream, int32_t* lines_out) {
  moe::clear_error();
  if (!r || (n > 0 && !experts) || n < 0) return set_error(MOE_ERR_INVALID, "bad arguments");
  return moe::ring_stage(r, layer_id, experts, n, static_cast<hipStream_t>(copy_stream),
                         lines_out);
}

moe_status moe_ring_prefetch(moe_ring* r, int32_t layer_id, const int32_t* experts, int32_t n,
                             void* copy_stream) {
  moe::clear_error();
  if (!r || (n > 0 && !experts) || n < 0) return set_error(MOE_ERR_INVALID, "bad arguments");
  return moe::ring_stage(r, layer_id, experts, n, static_cast<hipStream_t>(copy_stream),
                         nullptr, nullptr, false, MOE_COPY_CROSS_LAYER, /*hold=*/false);
}

moe_status moe_ring_wait_ready(moe_ring* r, const int32_t* lines, int32_t n, void* stream) {
  moe::clear_error();
  if (!r || (n > 0 && !lines) || n < 0) return set_error(MOE_ERR_INVALID, "bad arguments");
  return moe::ring_wait_ready(r, lines, n, static_cast<hipStream_t>(stream));
}

moe_status moe_ring_release(moe_ring* r, const int32_t* lines, int32_t n, void* stream) {
  moe::clear_error();
  if (!r || (n > 0 && !lines) || n < 0) return set_error(MOE_ERR_INVALID, "bad arguments");
  return moe::ring_release(r, lines, n, static_cast<hipStream_t>(stream));
}

const void* moe_ring_line_ptr(const moe_ring* r, int32_t line) {
  if (!r || line < 0 || line >= r->n_lines) return nullptr;
  return r->lines + static_cast<size_t>(line) * r->line_bytes;
}

moe_status moe_ring_stats(const moe_ring* r, moe_ring_stats_t* out) {
  moe::clear_error();
  if (!r || !out) return set_error(MOE_ERR_INVALID, "bad arguments");
  *out = r->stats;
  return MOE_OK;
}

moe_status moe_ring_reset_stats(moe_ring* r) {
  moe::clear_error();
  if (!r) return set_error(MOE_ERR_INVALID, "ring is NULL");
  const int32_t nl = r->stats.n_lines;
  r->stats = moe_ring_stats_t{};
  r->stats.version = 3;
  r->stats.n_lines = nl;
  return MOE_OK;
}

moe_status moe_ring_invalidate(moe_ring* r) {
  moe::clear_error();
  if (!r) return set_error(MOE_ERR_INVALID, "ring is NULL");
  r->where.clear();
  for (auto& ln : r->line) {
    ln.layer = -1;
    ln.expert = -1;
    ln.last_use = 0;
  }
  return MOE_OK;
}

void moe_ring_destroy(moe_ring* r) {
  if (!r) return;
  for (size_t l = 0; l < r->line.size(); ++l) {
    if (r->line[l].has_ready) (void)hipEventSynchronize(r->ready[l]);
    if (r->line[l].has_release) (void)hipEventSynchronize(r->release[l]);
  }
  for (hipEvent_t e : r->ready) (void)hipEventDestroy(e);
  for (hipEvent_t e : r->release) (void)hipEventDestroy(e);
  if (r->copy2) {
    (void)hipStreamSynchronize(r->copy2);
    (void)hipStreamDestroy(r->copy2);
  }
  delete r;
}

}  // extern "C"
