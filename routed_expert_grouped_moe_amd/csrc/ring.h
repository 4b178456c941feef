// Host-side state of a ring of device expert lines (the opaque moe_ring of the ABI).
#pragma once

#include <unordered_map>
#include <vector>

#include "moe_internal.h"

struct moe_ring {
  struct Line {
    int32_t layer = -1;           // (layer, expert) held, or -1
    int32_t expert = -1;
    uint64_t last_use = 0;        // LRU clock of the last staging that used the line
    bool held = false;            // handed out by a staging call, not yet released
    bool has_ready = false;       // `ready` has been recorded at least once
    bool has_release = false;     // `release` has been recorded at least once
    uint64_t release_seq = 0;     // release epoch (per ring, increasing in record order)
    hipStream_t release_stream = nullptr;
    // A stream that has waited for the line's latest fill (its `ready`), or NULL. A release
    // recorded on another stream first waits for that fill, so that a later copy into the
    // line, which waits only for the release, cannot overtake the fill.
    hipStream_t ready_seen = nullptr;
    bool ready_seen_valid = false;
  };
  struct Bank {
    const char* base = nullptr;
    // The device's address of the pinned bank (hipHostGetDevicePointer), when it has one and
    // it is 16-byte aligned: misses are then copied by the library's copy kernel, else by
    // hipMemcpyAsync.
    const char* dev_base = nullptr;
    std::vector<int32_t> slot;    // bank slot of each expert, -1 = resident
  };

  moe_shape shape{};
  size_t line_bytes = 0;
  char* lines = nullptr;
  int32_t n_lines = 0;
  std::vector<Line> line;
  std::vector<hipEvent_t> ready, release;
  std::unordered_map<int64_t, int32_t> where;   // (layer << 32 | expert) -> line
  std::unordered_map<int32_t, Bank> banks;
  uint64_t clock = 0;
  uint64_t sweeps = 0;            // chunk passes planned; odd passes walk experts downward
  uint64_t release_counter = 0;
  // Release-epoch coalescing, per copy stream: copy stream `copy` has already waited for
  // every release recorded on `rel` up to epoch `seq`, so older releases need no wait.
  struct Coal {
    hipStream_t rel = nullptr, copy = nullptr;
    uint64_t seq = 0;
  };
  Coal coal[2];
  // Library-owned second copy stream (default priority, created on first use): the chunk
  // sequencer alternates a wave's copies between it and the caller's copy stream, so one
  // copy's per-transfer set-up overlaps the other's transfer.
  hipStream_t copy2 = nullptr;
  moe_ring_stats_t stats{};
};

namespace moe {

inline int64_t ring_key(int32_t layer, int32_t expert) {
  return (static_cast<int64_t>(layer) << 32) | static_cast<uint32_t>(expert);
}

// Implementations of the ABI calls, used by the chunk sequencer too (no argument checks
// beyond the ring's own; set the thread's last error on failure).
// two_streams: misses alternate between copy_stream and the ring's own second copy stream.
// later (optional, indexed by expert of `layer`): experts that further stagings of the same
// pass will ask for. A miss then evicts, least recently used first, a line that holds none of
// them when there is one (a near-Belady choice for the known rest of the pass), else the least
// recently used line.
// kind: MOE_COPY_* category the staging's requested and copied bytes are counted under.
// hold: the lines stay held until ring_release (else each miss's release is recorded on its
// copy stream right behind the copy, and no line stays held).
// kernel_copy: misses are copied by the library's copy kernel (when the bank has a device
// mapping) instead of hipMemcpyAsync.
MOE_HIDDEN moe_status ring_stage(moe_ring* r, int32_t layer, const int32_t* experts, int32_t n,
                                 hipStream_t copy_stream, int32_t* lines_out,
                                 const std::vector<char>* later = nullptr,
                                 bool two_streams = false, int kind = MOE_COPY_DEMAND,
                                 bool hold = true, bool kernel_copy = false);
MOE_HIDDEN moe_status ring_wait_ready(moe_ring* r, const int32_t* lines, int32_t n,
                                      hipStream_t stream);
MOE_HIDDEN moe_status ring_release(moe_ring* r, const int32_t* lines, int32_t n,
                                   hipStream_t stream);

// thread-local error text
MOE_HIDDEN const char* last_error_text();
MOE_HIDDEN void clear_error();
MOE_HIDDEN moe_status set_error(moe_status s, const char* fmt, ...)
    __attribute__((format(printf, 2, 3)));

}  // namespace moe
