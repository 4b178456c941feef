// CPU check of the ring's bookkeeping (csrc/ring.hip compiled with g++ against the host
// stand-in hip/hip_runtime.h, under AddressSanitizer and UndefinedBehaviorSanitizer).
//
// Streams and events are simulated with vector clocks: an operation enqueued on a stream
// happens after everything the stream already holds and everything any event it waited for
// covered. Copies into ring lines (hipMemcpyAsync) and reads of ring lines (the driver's stand-in
// for the GEMMs that read a staged expert between moe_ring_wait_ready and moe_ring_release) are
// logged, and checked:
//   - the copy that last filled a read's line (in host order) brought the expert the read
//     expects, and happens before the read;
//   - every later copy into the same line happens after the read (the copy waited for it);
//   - the copies into one line are ordered among themselves (a refill cannot overtake the
//     fill before it).
//
// Modes (argv[1]):
//   random <seed> <steps>     random stagings on two copy streams, reads on two compute
//                             streams, releases on either stream (some without waiting for the
//                             fill) (including a line read and released on one stream, then
//                             found as a hit and released on the other), and prefetches
//   two_streams               the fixed sequence of the last case
//   model <file>              replay staging waves written by tests/ring_model.py through the
//                             internal staging call, and print the hit and miss counts
// Exit status 0 when every check passes; the first failure is printed.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <map>
#include <random>
#include <string>
#include <vector>

#include "hip/hip_runtime.h"
#include "../../routed_expert_grouped_moe_amd/csrc/ring.h"

namespace {

constexpr int kMaxStreams = 32;
typedef std::vector<uint64_t> VC;

struct Op {
  int stream;
  VC vc;
  const char* src;     // copy: bank address written; read: bank address expected
  bool is_copy;
  uint64_t seq;        // host issue order
};

uint64_t g_seq = 0;
int g_fail = 0;
std::map<const void*, std::vector<Op>> g_ops;   // per ring line address

}  // namespace

struct SimStream {
  int id;
  VC vc = VC(kMaxStreams, 0);
};
struct SimEvent {
  VC vc = VC(kMaxStreams, 0);
  bool recorded = false;
};

namespace {
std::vector<SimStream*> g_streams;

SimStream* stream_of(hipStream_t s) {
  if (s) return s;
  static SimStream null_stream{0};                // the default stream
  return &null_stream;
}

Op enqueue(hipStream_t hs, const char* src, bool is_copy) {
  SimStream* s = stream_of(hs);
  s->vc[s->id]++;
  return Op{s->id, s->vc, src, is_copy, ++g_seq};
}

bool hb(const Op& a, const Op& b) { return a.vc[a.stream] <= b.vc[a.stream]; }

void fail(const char* what, const void* line, const Op& a, const Op& b) {
  if (g_fail++ < 5)
    fprintf(stderr, "RACE %s: line %p, ops #%llu (stream %d) and #%llu (stream %d)\n", what,
            line, (unsigned long long)a.seq, a.stream, (unsigned long long)b.seq, b.stream);
}

void check_all() {
  for (auto& kv : g_ops) {
    const std::vector<Op>& ops = kv.second;
    const Op* prev_copy = nullptr;           // copies into one line must be ordered
    for (size_t i = 0; i < ops.size(); ++i) {
      if (!ops[i].is_copy) continue;
      if (prev_copy && !hb(*prev_copy, ops[i])) fail("copy not after the line's previous copy", kv.first, *prev_copy, ops[i]);
      prev_copy = &ops[i];
    }
    for (size_t i = 0; i < ops.size(); ++i) {
      if (ops[i].is_copy) continue;
      const Op& r = ops[i];
      const Op* w = nullptr;
      for (size_t j = 0; j < i; ++j)
        if (ops[j].is_copy) w = &ops[j];
      if (!w) { fail("read of a line never filled", kv.first, r, r); continue; }
      if (w->src != r.src) fail("read finds another expert", kv.first, *w, r);
      else if (!hb(*w, r)) fail("read not after its copy", kv.first, *w, r);
      for (size_t j = i + 1; j < ops.size(); ++j)
        if (ops[j].is_copy && !hb(r, ops[j])) fail("copy not after an earlier read", kv.first, r, ops[j]);
    }
  }
}

}  // namespace

// ---------------------------------------------------------------- the HIP stand-in

const char* hipGetErrorString(hipError_t) { return "simulated error"; }
hipError_t hipGetLastError(void) { return hipSuccess; }
hipError_t hipStreamCreateWithFlags(hipStream_t* s, unsigned) {
  static int next_id = 1;                          // 0 is the default stream's
  if (next_id >= kMaxStreams) return hipErrorOutOfMemory;
  SimStream* n = new SimStream();
  n->id = next_id++;
  g_streams.push_back(n);
  *s = n;
  return hipSuccess;
}
hipError_t hipStreamDestroy(hipStream_t s) {
  auto it = std::find(g_streams.begin(), g_streams.end(), s);
  if (it == g_streams.end()) return hipErrorInvalidValue;
  g_streams.erase(it);
  delete s;
  return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
hipError_t hipStreamWaitEvent(hipStream_t hs, hipEvent_t e, unsigned) {
  if (!e) return hipErrorInvalidValue;
  SimStream* s = stream_of(hs);
  if (e->recorded)
    for (int i = 0; i < kMaxStreams; ++i) s->vc[i] = std::max(s->vc[i], e->vc[i]);
  return hipSuccess;
}
hipError_t hipEventCreateWithFlags(hipEvent_t* e, unsigned) {
  *e = new SimEvent();
  return hipSuccess;
}
hipError_t hipEventDestroy(hipEvent_t e) {
  delete e;
  return hipSuccess;
}
hipError_t hipEventRecord(hipEvent_t e, hipStream_t hs) {
  if (!e) return hipErrorInvalidValue;
  e->vc = stream_of(hs)->vc;
  e->recorded = true;
  return hipSuccess;
}
hipError_t hipEventSynchronize(hipEvent_t) { return hipSuccess; }
hipError_t hipMemcpyAsync(void* dst, const void* src, size_t, hipMemcpyKind, hipStream_t s) {
  g_ops[dst].push_back(enqueue(s, static_cast<const char*>(src), true));
  return hipSuccess;
}
// Pinned memory is mapped at its host address (the library then copies with its kernel).
hipError_t hipHostGetDevicePointer(void** dev, void* host, unsigned) {
  *dev = host;
  return hipSuccess;
}
namespace moe {
hipError_t launch_line_copy(void* dst, const void* src_dev, size_t bytes, hipStream_t s) {
  return hipMemcpyAsync(dst, src_dev, bytes, hipMemcpyHostToDevice, s);
}
}  // namespace moe

// moe_ring_create sizes a line from the shape after checking it; the shape checks live with
// the workspace layout in the GPU part of the library, so this check stands in for them.
extern "C" size_t moe_workspace_bytes(const moe_shape* s, int64_t) {
  return (s && s->d > 0 && s->inter > 0 && s->n_experts > 0) ? 1 : 0;
}

// ---------------------------------------------------------------- driver

namespace {

struct World {
  moe_shape sh{64, 0, 1, 64, 0, MOE_BF16};
  moe_ring* ring = nullptr;
  std::vector<char> lines_mem, bank_mem;
  char* lines = nullptr;
  const char* bank = nullptr;
  size_t line_bytes = 0;
  int E = 0;

  World(int n_lines, int experts) : E(experts) {
    sh.n_experts = experts;
    line_bytes = 3ull * sh.inter * sh.d * 2;
    lines_mem.resize(line_bytes * n_lines + 256);
    bank_mem.resize(line_bytes * experts);
    uintptr_t p = reinterpret_cast<uintptr_t>(lines_mem.data());
    lines = reinterpret_cast<char*>((p + 255) & ~uintptr_t(255));
    bank = bank_mem.data();
    if (moe_ring_create(&sh, lines, n_lines, &ring) != MOE_OK) {
      fprintf(stderr, "ring create failed: %s\n", moe::last_error_text());
      exit(2);
    }
    std::vector<int32_t> slot(experts);
    for (int e = 0; e < experts; ++e) slot[e] = e;
    if (moe_ring_bind_bank(ring, 0, bank, slot.data()) != MOE_OK) exit(2);
  }
  ~World() { moe_ring_destroy(ring); }
  const char* expert_src(int e) const { return bank + static_cast<size_t>(e) * line_bytes; }
  void read(hipStream_t s, int line, int expert) {
    const void* addr = moe_ring_line_ptr(ring, line);
    g_ops[addr].push_back(enqueue(s, expert_src(expert), false));
  }
};

int run_random(unsigned seed, int steps) {
  World w(6, 14);
  std::mt19937 rng(seed);
  hipStream_t copy[2], comp[2];
  hipStreamCreateWithFlags(&copy[0], 0);
  hipStreamCreateWithFlags(&copy[1], 0);
  hipStreamCreateWithFlags(&comp[0], 0);
  hipStreamCreateWithFlags(&comp[1], 0);
  struct Held {
    int line, expert;
  };
  std::vector<Held> held;
  for (int step = 0; step < steps; ++step) {
    const int op = static_cast<int>(rng() % 10);
    if (op < 5) {                              // stage 1..3 distinct experts
      std::vector<int32_t> ex;
      const int n = 1 + static_cast<int>(rng() % 3);
      while (static_cast<int>(ex.size()) < n) {
        const int e = static_cast<int>(rng() % w.E);
        bool dup = std::find(ex.begin(), ex.end(), e) != ex.end();
        for (const Held& h : held) dup |= h.expert == e;   // not staged twice while held
        if (!dup) ex.push_back(e);
        if (ex.size() + held.size() >= 6) break;
      }
      if (ex.empty()) continue;
      std::vector<int32_t> out(ex.size());
      const moe_status st = moe_stage_experts(w.ring, 0, ex.data(), static_cast<int32_t>(ex.size()),
                                              copy[rng() % 2], out.data());
      if (st == MOE_ERR_RING) continue;        // too few free lines: nothing changed
      if (st != MOE_OK) { fprintf(stderr, "stage: %s\n", moe::last_error_text()); return 2; }
      for (size_t i = 0; i < ex.size(); ++i) held.push_back({out[i], ex[i]});
    } else if (op < 8 && !held.empty()) {      // one compute stream reads some and releases
      hipStream_t s = comp[rng() % 2];
      const size_t take = 1 + rng() % held.size();
      std::vector<int32_t> ls;
      for (size_t i = 0; i < take; ++i) ls.push_back(held[i].line);
      // some holders release without waiting for the fill, and then never read
      const bool waits = rng() % 5 != 0;
      if (waits &&
          moe_ring_wait_ready(w.ring, ls.data(), static_cast<int32_t>(ls.size()), s) != MOE_OK)
        return 2;
      for (size_t i = 0; i < take; ++i)
        if (waits && rng() % 4) w.read(s, held[i].line, held[i].expert);   // some never read
      if (moe_ring_release(w.ring, ls.data(), static_cast<int32_t>(ls.size()), s) != MOE_OK) return 2;
      held.erase(held.begin(), held.begin() + static_cast<long>(take));
    } else {                                   // prefetch an expert that is not held
      const int32_t e = static_cast<int32_t>(rng() % w.E);
      bool dup = false;
      for (const Held& h : held) dup |= h.expert == e;
      if (dup) continue;
      const moe_status st = moe_ring_prefetch(w.ring, 0, &e, 1, copy[rng() % 2]);
      if (st != MOE_OK && st != MOE_ERR_RING) { fprintf(stderr, "prefetch: %s\n", moe::last_error_text()); return 2; }
    }
  }
  moe_ring_stats_t stats;
  moe_ring_stats(w.ring, &stats);
  int64_t req = 0, cop = 0;
  for (int k = 0; k < MOE_COPY_KINDS; ++k) {
    req += stats.requested_bytes[k];
    cop += stats.copied_bytes[k];
  }
  if (cop != stats.bytes_h2d || req != (stats.hits + stats.misses) * static_cast<int64_t>(w.line_bytes)) {
    fprintf(stderr, "copy categories do not reconcile: copied %lld of %lld, requested %lld\n",
            (long long)cop, (long long)stats.bytes_h2d, (long long)req);
    return 1;
  }
  check_all();
  printf("random seed %u: %d steps, %lld hits, %lld misses, %d races\n", seed, steps,
         (long long)stats.hits, (long long)stats.misses, g_fail);
  return g_fail ? 1 : 0;
}

int run_two_streams() {
  // A line read and released on stream A, staged again as a hit and released on stream B
  // without being read there, then evicted by a miss: the miss's copy must wait for A's read.
  World w(1, 4);
  hipStream_t copy_s, a, b;
  hipStreamCreateWithFlags(&copy_s, 0);
  hipStreamCreateWithFlags(&a, 0);
  hipStreamCreateWithFlags(&b, 0);
  int32_t e0 = 0, e1 = 1, l = -1;
  if (moe_stage_experts(w.ring, 0, &e0, 1, copy_s, &l) != MOE_OK) return 2;
  moe_ring_wait_ready(w.ring, &l, 1, a);
  w.read(a, l, e0);
  moe_ring_release(w.ring, &l, 1, a);
  if (moe_stage_experts(w.ring, 0, &e0, 1, copy_s, &l) != MOE_OK) return 2;   // a hit
  moe_ring_wait_ready(w.ring, &l, 1, b);
  moe_ring_release(w.ring, &l, 1, b);
  if (moe_stage_experts(w.ring, 0, &e1, 1, copy_s, &l) != MOE_OK) return 2;   // evicts e0
  moe_ring_wait_ready(w.ring, &l, 1, a);
  w.read(a, l, e1);
  moe_ring_release(w.ring, &l, 1, a);
  check_all();
  printf("two streams: %d races\n", g_fail);
  return g_fail ? 1 : 0;
}

int run_model(const char* path) {
  // Lines: "ring <n_lines> <n_experts>", then "stage <kind> <n> e... | later <m> e...",
  // "release <n> e...". Stages go through the internal call the chunk sequencer uses, with the
  // model's `later` set, on alternating copy streams; releases name experts of staged waves.
  FILE* f = fopen(path, "r");
  if (!f) return 2;
  int n_lines = 0, E = 0;
  if (fscanf(f, " ring %d %d", &n_lines, &E) != 2) return 2;
  World w(n_lines, E);
  hipStream_t copy_s, comp;
  hipStreamCreateWithFlags(&copy_s, 0);
  hipStreamCreateWithFlags(&comp, 0);
  std::map<int, int> line_of;
  char word[32];
  while (fscanf(f, " %31s", word) == 1) {
    if (!strcmp(word, "stage")) {
      int kind = 0, n = 0, m = 0;
      if (fscanf(f, " %d %d", &kind, &n) != 2) return 2;
      std::vector<int32_t> ex(n), out(n);
      for (int i = 0; i < n; ++i)
        if (fscanf(f, " %d", &ex[i]) != 1) return 2;
      if (fscanf(f, " later %d", &m) != 1) return 2;
      std::vector<char> later(E, 0);
      for (int i = 0; i < m; ++i) {
        int e;
        if (fscanf(f, " %d", &e) != 1) return 2;
        later[e] = 1;
      }
      const moe_status st = moe::ring_stage(w.ring, 0, ex.data(), n, copy_s, out.data(), &later,
                                            /*two_streams=*/true, kind);
      if (st == MOE_ERR_RING) { printf("stage refused\n"); continue; }
      if (st != MOE_OK) return 2;
      for (int i = 0; i < n; ++i) line_of[ex[i]] = out[i];
    } else if (!strcmp(word, "release")) {
      int n = 0;
      if (fscanf(f, " %d", &n) != 1) return 2;
      std::vector<int32_t> ls(n), es(n);
      for (int i = 0; i < n; ++i) {
        if (fscanf(f, " %d", &es[i]) != 1) return 2;
        ls[i] = line_of.at(es[i]);
      }
      moe_ring_wait_ready(w.ring, ls.data(), n, comp);
      for (int i = 0; i < n; ++i) w.read(comp, ls[i], es[i]);
      moe_ring_release(w.ring, ls.data(), n, comp);
    } else {
      return 2;
    }
  }
  fclose(f);
  moe_ring_stats_t st;
  moe_ring_stats(w.ring, &st);
  check_all();
  printf("model hits %lld misses %lld copied", (long long)st.hits, (long long)st.misses);
  for (int k = 0; k < MOE_COPY_KINDS; ++k) printf(" %lld", (long long)(st.copied_bytes[k] / static_cast<int64_t>(w.line_bytes)));
  printf(" races %d\n", g_fail);
  return g_fail ? 1 : 0;
}

}  // namespace

int main(int argc, char** argv) {
  int rc = 2;
  if (argc >= 2 && !strcmp(argv[1], "random") && argc == 4)
    rc = run_random(static_cast<unsigned>(atoi(argv[2])), atoi(argv[3]));
  else if (argc >= 2 && !strcmp(argv[1], "two_streams"))
    rc = run_two_streams();
  else if (argc == 3 && !strcmp(argv[1], "model"))
    rc = run_model(argv[2]);
  else
    fprintf(stderr, "usage: %s random <seed> <steps> | two_streams | model <file>\n", argv[0]);
  for (SimStream* s : g_streams) delete s;      // the driver's own streams
  g_streams.clear();
  return rc;
}
