// C ABI entry points: argument checks, workspace layout and the launch sequence of one
// routed MoE layer (route, then expert-major chunks).
#include <string.h>

#include <algorithm>
#include <unordered_map>
#include <vector>

#include <atomic>

#include "ring.h"

namespace moe {

namespace {

std::atomic<int32_t> g_opt_fused_gu_down{0};

constexpr size_t kAlign = 256;
inline size_t align_up(size_t v) { return (v + kAlign - 1) & ~(kAlign - 1); }
inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
inline size_t elt_bytes(int dtype) { return dtype == MOE_BF16 ? 2 : 4; }

moe_status check_shape(const moe_shape* sh) {
  if (!sh) return set_error(MOE_ERR_INVALID, "shape is NULL");
  if (sh->d < 64 || sh->d > 16384 || sh->d % 64)
    return set_error(MOE_ERR_INVALID, "d=%d must be a multiple of 64 in [64, 16384]", sh->d);
  if (sh->n_experts < 1 || sh->n_experts > 1024)
    return set_error(MOE_ERR_INVALID, "n_experts=%d must be in [1, 1024]", sh->n_experts);
  if (sh->top_k < 1 || sh->top_k > sh->n_experts)
    return set_error(MOE_ERR_INVALID, "top_k=%d must be in [1, n_experts]", sh->top_k);
  if (sh->inter < 64 || sh->inter > 16384 || sh->inter % 64)
    return set_error(MOE_ERR_INVALID, "inter=%d must be a multiple of 64 in [64, 16384]",
                     sh->inter);
  if (sh->inter_shared < 0 || sh->inter_shared > 65536 || sh->inter_shared % 64)
    return set_error(MOE_ERR_INVALID, "inter_shared=%d must be a multiple of 64 in [0, 65536]",
                     sh->inter_shared);
  if (sh->dtype != MOE_BF16 && sh->dtype != MOE_F32)
    return set_error(MOE_ERR_INVALID, "dtype=%d", sh->dtype);
  return MOE_OK;
}

moe_status check_layer(const moe_layer* L) {
  if (!L) return set_error(MOE_ERR_INVALID, "layer is NULL");
  moe_status st = check_shape(&L->shape);
  if (st != MOE_OK) return st;
  const moe_shape& sh = L->shape;
  if (!L->w_router || !aligned(L->w_router, 16))
    return set_error(MOE_ERR_INVALID, "w_router NULL or not 16-byte aligned");
  if (L->router_bias && !aligned(L->router_bias, 4))
    return set_error(MOE_ERR_INVALID, "router_bias not 4-byte aligned");
  if (sh.inter_shared > 0) {
    if (!L->w_gu_shared || !L->w_down_shared || !aligned(L->w_gu_shared, 16) ||
        !aligned(L->w_down_shared, 16))
      return set_error(MOE_ERR_INVALID, "shared expert weights NULL or not 16-byte aligned");
  }
  return MOE_OK;
}

// Expert table checks (needed by the chunk calls only). Sets *offloaded when some expert
// comes from the ring.
moe_status check_experts(const moe_layer* L, bool* offloaded) {
  *offloaded = false;
  if (!L->expert_lines) return set_error(MOE_ERR_INVALID, "expert_lines is NULL");
  const moe_ring::Bank* bank = nullptr;
  if (L->ring) {
    if (L->layer_id < 0) return set_error(MOE_ERR_INVALID, "layer_id=%d", L->layer_id);
    auto it = L->ring->banks.find(L->layer_id);
    if (it != L->ring->banks.end()) bank = &it->second;
    const moe_shape& a = L->ring->shape;
    const moe_shape& b = L->shape;
    if (a.d != b.d || a.inter != b.inter || a.dtype != b.dtype || a.n_experts != b.n_experts)
      return set_error(MOE_ERR_RING, "ring shape does not match the layer");
  }
  for (int e = 0; e < L->shape.n_experts; ++e) {
    const void* p = L->expert_lines[e];
    if (p) {
      if (!aligned(p, 16)) return set_error(MOE_ERR_INVALID, "expert line %d not aligned", e);
      continue;
    }
    if (!bank) return set_error(MOE_ERR_RING, "expert %d has no device line and no ring bank", e);
    if (bank->slot[e] < 0)
      return set_error(MOE_ERR_RING, "expert %d has no device line and is not in the bank", e);
    *offloaded = true;
  }
  return MOE_OK;
}

// A side stream for work that may run beside the caller's stream, with a fork event (the
// side stream waits for everything the caller enqueued before it) and a done event (the
// caller's stream waits for the side work). One set per host thread and device, created on
// first use and kept for the life of the thread; default priority.
struct SideStream {
  hipStream_t stream = nullptr;
  hipEvent_t fork_ev = nullptr;
  hipEvent_t done_ev = nullptr;

  hipError_t acquire() {
    struct Entry {
      hipStream_t s = nullptr;
      hipEvent_t f = nullptr, d = nullptr;
    };
    thread_local std::unordered_map<int, Entry> cache;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    Entry& en = cache[dev];
    if (!en.s) {
      e = hipStreamCreateWithFlags(&en.s, hipStreamNonBlocking);
      if (e != hipSuccess) { en.s = nullptr; return e; }
    }
    if (!en.f) {
      e = hipEventCreateWithFlags(&en.f, hipEventDisableTiming);
      if (e != hipSuccess) { en.f = nullptr; return e; }
    }
    if (!en.d) {
      e = hipEventCreateWithFlags(&en.d, hipEventDisableTiming);
      if (e != hipSuccess) { en.d = nullptr; return e; }
    }
    stream = en.s;
    fork_ev = en.f;
    done_ev = en.d;
    return hipSuccess;
  }
  hipError_t fork(hipStream_t s) {
    hipError_t e = acquire();
    if (e == hipSuccess) e = hipEventRecord(fork_ev, s);
    if (e == hipSuccess) e = hipStreamWaitEvent(stream, fork_ev, 0);
    return e;
  }
  hipError_t record_done() { return hipEventRecord(done_ev, stream); }
  hipError_t join(hipStream_t s) { return hipStreamWaitEvent(s, done_ev, 0); }
};

// Joins the side work into the caller's stream on every early return after it was forked, so
// the caller's stream never runs ahead of work that still writes the workspace.
struct JoinOnExit {
  SideStream& side;
  hipStream_t s;
  bool armed = false;
  ~JoinOnExit() {
    if (armed) (void)side.join(s);
  }
  hipError_t join() {
    armed = false;
    return side.join(s);
  }
};

// True when line e is at lines[0] + e * stride for every e (one block of E lines).
bool uniform_lines(const void* const* lines, int E, int64_t* stride) {
  const uintptr_t b = reinterpret_cast<uintptr_t>(lines[0]);
  const uintptr_t st = E > 1 ? reinterpret_cast<uintptr_t>(lines[1]) - b : 0;
  for (int e = 0; e < E; ++e)
    if (reinterpret_cast<uintptr_t>(lines[e]) != b + static_cast<uintptr_t>(e) * st) return false;
  *stride = static_cast<int64_t>(st);
  return true;
}

#define MOE_HIP(call)                                                                      \
  do {                                                                                     \
    hipError_t e_ = (call);                                                                \
    if (e_ != hipSuccess)                                                                  \
      return set_error(MOE_ERR_HIP, "%s: %s", #call, hipGetErrorString(e_));               \
  } while (0)

// counts_in_chunks: the caller's chunk loop fills chunk_counts (each chunk's bucketing writes
// its row), so the per-chunk histogram is not launched here.
moe_status route_impl(const moe_layer* L, const void* x, int64_t T, int64_t chunk,
                      int32_t* ids, float* weights, int32_t* chunk_counts, float* logits,
                      hipStream_t s, bool counts_in_chunks = false) {
  const moe_shape& sh = L->shape;
  MOE_HIP(launch_router_gemm(sh.dtype, x, L->w_router, L->router_bias, T, sh.d, sh.n_experts,
                             logits, s));
  const int64_t n_cc = (T + chunk - 1) / chunk * sh.n_experts;
  if (topk_counts_fused(T)) {
    MOE_HIP(launch_topk_counts_small(logits, T, sh.n_experts, sh.top_k, ids, weights, chunk,
                                     chunk_counts, n_cc, s));
    return MOE_OK;
  }
  MOE_HIP(launch_topk(logits, T, sh.n_experts, sh.top_k, ids, weights, chunk_counts,
                      counts_in_chunks ? 0 : n_cc, s));
  if (!counts_in_chunks)
    MOE_HIP(launch_chunk_hist(ids, T, sh.top_k, sh.n_experts, chunk, chunk_counts, s));
  return MOE_OK;
}

// Shares of the ring's lines a layer call may pin, in sixteenths. On the 8-layer stack
// (Zipf 1.5, 128 lines) allowing 14/16 and 15/16 besides 0..12/16 took a pass from
// 1,182-1,189 to 1,147-1,154 and 1,127-1,139 ms: fewer bytes, though in more, smaller waves.
constexpr int kPinSixteenths[] = {0, 4, 8, 12, 14, 15};
// A wave (a staging with its GEMM launches) costs about an eighth of a line copy in the
// same measurement (953 more waves per pass for 258 fewer copies saved 12-20 ms); the
// estimate weighs copies by 8 and waves by 1.
constexpr int64_t kCopyPerWave = 8;
constexpr int kPinChoices = sizeof(kPinSixteenths) / sizeof(kPinSixteenths[0]);

// Experts held in the ring for a whole layer call, and their lines.
struct Pinned {
  std::vector<int32_t> experts;   // ascending
  std::vector<int32_t> lines;
};

// Cost of a layer call if the H experts used by the most chunks (by_freq[0..H)) stayed pinned
// and the others streamed through the remaining cap lines, least recently used first, each
// chunk pass walking its experts upward or downward in turn from sweep0, in waves of cap/2:
// kCopyPerWave per copy plus one per wave (holds ignored: an estimate for choosing H, not the
// ring's exact count). The lines' experts form a recency list (most recent first), so a
// lookup or an eviction is O(1): the call is planned on the host while the GPU waits.
int64_t estimate_cost(const std::vector<std::vector<int32_t>>& used,
                      const std::vector<int32_t>& by_freq, int H, int cap, uint64_t sweep0,
                      int E) {
  std::vector<char> hot(E, 0), in(E, 0);
  for (int i = 0; i < H; ++i) hot[by_freq[i]] = 1;
  std::vector<int32_t> prv(E, -1), nxt(E, -1);
  int head = -1, tail = -1, resident = 0;
  auto unlink = [&](int e) {
    (prv[e] >= 0 ? nxt[prv[e]] : head) = nxt[e];
    (nxt[e] >= 0 ? prv[nxt[e]] : tail) = prv[e];
  };
  auto push_front = [&](int e) {
    prv[e] = -1;
    nxt[e] = head;
    (head >= 0 ? prv[head] : tail) = e;
    head = e;
  };
  int64_t copies = H, waves = 0;
  const int per_wave = std::max(1, cap / 2);
  for (size_t c = 0; c < used.size(); ++c) {
    const std::vector<int32_t>& u = used[c];
    const bool down = ((sweep0 + c) & 1) != 0;
    int streamed = 0;
    for (int e : u) streamed += hot[e] ? 0 : 1;
    waves += std::max(1, (streamed + per_wave - 1) / per_wave);
    for (size_t i = 0; i < u.size(); ++i) {
      const int e = u[down ? u.size() - 1 - i : i];
      if (hot[e]) continue;
      if (in[e]) {
        unlink(e);
      } else {
        ++copies;
        if (resident == cap) {                 // evict the least recently used
          const int v = tail;
          unlink(v);
          in[v] = 0;
          --resident;
        }
        in[e] = 1;
        ++resident;
      }
      push_front(e);
    }
  }
  return kCopyPerWave * copies + waves;
}

// The experts of a layer call to pin: H = n_lines * kPinSixteenths / 16, the most chunks'
// experts first (ties to the lower id), H chosen by estimate_cost (ties to the smaller H).
// A skewed routing, whose hot experts recur in every chunk, keeps them in the ring for the
// call instead of streaming them in and out once per chunk; a uniform one pins nothing.
std::vector<int32_t> choose_pinned(const moe_layer* L, const int32_t* hc, int64_t n_chunks) {
  const int E = L->shape.n_experts;
  const int n = L->ring->n_lines;
  std::vector<std::vector<int32_t>> used(static_cast<size_t>(n_chunks));
  std::vector<int32_t> freq(E, 0);
  for (int64_t c = 0; c < n_chunks; ++c)
    for (int e = 0; e < E; ++e)
      if (!L->expert_lines[e] && hc[c * E + e] > 0) {
        used[c].push_back(e);
        ++freq[e];
      }
  std::vector<int32_t> by_freq;
  for (int e = 0; e < E; ++e)
    if (freq[e] > 0) by_freq.push_back(e);
  std::stable_sort(by_freq.begin(), by_freq.end(),
                   [&](int a, int b) { return freq[a] > freq[b]; });
  int best_h = 0;
  int64_t best = -1;
  for (int q = 0; q < kPinChoices; ++q) {
    const int H = std::min<int>(n * kPinSixteenths[q] / 16, static_cast<int>(by_freq.size()));
    if (q > 0 && H == 0) continue;
    const int64_t c = estimate_cost(used, by_freq, H, n - H, L->ring->sweeps, E);
    if (best < 0 || c < best) {
      best = c;
      best_h = H;
    }
  }
  std::vector<int32_t> pin(by_freq.begin(), by_freq.begin() + best_h);
  std::sort(pin.begin(), pin.end());
  return pin;
}

// The routed GEMMs of the M-tiles g covers: gate/up then down, or both in one fused launch
// when MOE_OPT_FUSED_GU_DOWN is on and the tiles allow it (the same h and Y bits).
hipError_t launch_routed(const moe_shape& sh, const void* x, int64_t t0, const GemmGroups& g,
                         const int32_t* row_tok, const int32_t* row_slot, void* h, float* y,
                         hipStream_t s) {
  if (g_opt_fused_gu_down.load(std::memory_order_relaxed) &&
      gu_down_fused_supported(sh.dtype, g.tile_rows, sh.inter))
    return launch_gu_down_fused(x, t0, sh.d, sh.inter, g, row_tok, row_slot, y, s);
  hipError_t err = launch_gu_routed(sh.dtype, x, t0, sh.d, sh.inter, g, row_tok, h, s);
  if (err == hipSuccess) err = launch_down_routed(sh.dtype, h, sh.d, sh.inter, g, row_slot, y, s);
  return err;
}

// Routed GEMMs of a chunk whose experts come partly from the ring: the chunk's used
// offloaded experts, in ascending id, are cut into waves of at most n_lines/2 experts; wave w
// covers the expert-id range [lo_w, hi_w) (resident experts in that range run with it). The
// waves run in ascending order on even passes of the ring and descending on odd ones
// (boustrophedon): the lines the last pass left behind are the first ones this pass asks for.
// The wave after the current one is staged on the copy stream before the current wave's GEMMs
// are enqueued, so copies overlap compute; each wave waits for its lines' `ready` events and
// then records their `release`. Misses evict lines this pass will not ask for again first.
// The order of the waves never changes a result bit: each expert's rows are computed alone
// and the combine sums in ascending expert id.
moe_status ring_waves(const moe_layer* L, const void* x, int64_t t0, int64_t n,
                      const int32_t* counts_host, char* ws, const WsLayout& W, hipStream_t s,
                      hipStream_t cs, const Pinned* pin) {
  const moe_shape& sh = L->shape;
  const int E = sh.n_experts, k = sh.top_k;
  moe_ring* R = L->ring;
  std::vector<int32_t> cnt(E);
  if (counts_host) {
    memcpy(cnt.data(), counts_host, sizeof(int32_t) * E);
  } else {
    MOE_HIP(hipMemcpyAsync(cnt.data(), ws + W.counts, sizeof(int32_t) * E,
                           hipMemcpyDeviceToHost, s));
    MOE_HIP(hipStreamSynchronize(s));
  }
  int64_t total = 0;
  for (int e = 0; e < E; ++e) {
    if (cnt[e] < 0) return set_error(MOE_ERR_INVALID, "negative count for expert %d", e);
    total += cnt[e];
  }
  if (total != n * k)
    return set_error(MOE_ERR_INVALID, "expert counts sum to %lld, chunk has %lld slots",
                     static_cast<long long>(total), static_cast<long long>(n * k));
  const int bm = routed_tile_rows(n, k, E);
  std::vector<int64_t> mt_begin(E + 1, 0);
  for (int e = 0; e < E; ++e) mt_begin[e + 1] = mt_begin[e] + mtiles_of(cnt[e], bm);

  std::vector<char> pinned(E, 0);
  const int n_pin = pin ? static_cast<int>(pin->experts.size()) : 0;
  for (int i = 0; i < n_pin; ++i) pinned[pin->experts[i]] = 1;
  std::vector<int32_t> used;
  bool all_offloaded = true;
  for (int e = 0; e < E; ++e) {
    all_offloaded &= L->expert_lines[e] == nullptr;
    if (!L->expert_lines[e] && cnt[e] > 0 && !pinned[e]) used.push_back(e);
  }
  // Misses are copied by the library's copy kernel when every routed expert of the layer is
  // offloaded: each wave's GEMMs then cover only the wave's experts and leave CUs free for the
  // copy workgroups, and kernel-to-kernel dependencies on the release events cost the link
  // nothing (6 MiB DMA copies behind such waits lose 10-45% of the link: 16,022 tokens through
  // 64 lines took 412-414 ms against 429-433 ms). With resident experts in the waves' ranges
  // the GEMMs fill the chip and the copy kernel would stall behind them (the 8-layer stack:
  // 1,141 ms against 1,113-1,119 ms with DMA copies), so those layers keep hipMemcpyAsync.
  // pinned experts sit in their held lines for the whole layer call and run with whichever
  // wave's expert-id range covers them, as resident experts do
  const int per_wave = std::max(1, (R->n_lines - n_pin) / 2);
  const int nw = std::max<int>(1, (static_cast<int>(used.size()) + per_wave - 1) / per_wave);
  std::vector<std::vector<int32_t>> wexp(nw), wlines(nw);
  std::vector<int32_t> lo(nw), hi(nw);
  const bool down = (R->sweeps++ & 1) != 0;
  for (int w = 0; w < nw; ++w) {
    const size_t b = static_cast<size_t>(w) * per_wave;
    const size_t e = std::min(used.size(), b + per_wave);
    for (size_t i = b; i < e; ++i) wexp[w].push_back(used[i]);
    if (down) std::reverse(wexp[w].begin(), wexp[w].end());
    wlines[w].resize(wexp[w].size());
    lo[w] = w == 0 ? 0 : hi[w - 1];
    hi[w] = (w + 1 < nw) ? used[static_cast<size_t>(w + 1) * per_wave] : E;
  }
  auto wave_at = [&](int i) { return down ? nw - 1 - i : i; };   // processing order
  std::vector<char> later(E, 0);
  for (int e : used) later[e] = 1;

  const void** wtab = reinterpret_cast<const void**>(ws + W.wtab);
  GemmGroups g{reinterpret_cast<const MTile*>(ws + W.mtiles),
               reinterpret_cast<const int32_t*>(ws + W.meta) + kMetaMTiles,
               reinterpret_cast<const int32_t*>(ws + W.offsets),
               reinterpret_cast<const int32_t*>(ws + W.counts), wtab, nullptr, 0, 0, 0, bm};
  const int32_t* row_tok = reinterpret_cast<const int32_t*>(ws + W.row_tok);
  const int32_t* row_slot = reinterpret_cast<const int32_t*>(ws + W.row_slot);
  char* h = ws + W.h;
  float* y = reinterpret_cast<float*>(ws + W.y);
  for (int i = 0; i < n_pin; ++i) R->stats.pinned_uses += cnt[pin->experts[i]] > 0 ? 1 : 0;
  if (n_pin > 0) {                             // this chunk's table entries of the pinned lines
    std::vector<const void*> pp(n_pin);
    for (int i = 0; i < n_pin; ++i) pp[i] = moe_ring_line_ptr(R, pin->lines[i]);
    moe_status pst = ring_wait_ready(R, pin->lines.data(), n_pin, s);
    if (pst != MOE_OK) return pst;
    MOE_HIP(launch_upload_pairs(wtab, pin->experts.data(), pp.data(), n_pin, s));
  }

  int staged = 0;                              // waves staged, in processing order
  moe_status st = MOE_OK;
  auto release_held = [&](int from) {          // unwind: give back lines of unfinished waves
    for (int i = from; i < staged; ++i) {
      const int w = wave_at(i);
      (void)ring_release(R, wlines[w].data(), static_cast<int32_t>(wlines[w].size()), s);
    }
  };
  for (int i = 0; i < nw; ++i) {
    const int w = wave_at(i);
    while (staged < nw && staged <= i + 1) {   // this wave, and the next one if lines allow
      const int ws_ = wave_at(staged);
      for (int e : wexp[ws_]) later[e] = 0;
      const int kind = staged == 0 ? MOE_COPY_INITIAL
                                   : (staged > i ? MOE_COPY_AHEAD : MOE_COPY_DEMAND);
      st = ring_stage(R, L->layer_id, wexp[ws_].data(), static_cast<int32_t>(wexp[ws_].size()),
                      cs, wlines[ws_].data(), &later, /*two_streams=*/true, kind,
                      /*hold=*/true, all_offloaded);
      if (st == MOE_ERR_RING && staged > i) { st = MOE_OK; break; }   // retry after release
      if (st != MOE_OK) { release_held(i); return st; }
      ++staged;
    }
    const int32_t nl = static_cast<int32_t>(wlines[w].size());
    std::vector<const void*> ptrs(nl);
    for (int i = 0; i < nl; ++i) ptrs[i] = moe_ring_line_ptr(R, wlines[w][i]);
    st = ring_wait_ready(R, wlines[w].data(), nl, s);
    hipError_t err = hipSuccess;
    if (st == MOE_OK) err = launch_upload_pairs(wtab, wexp[w].data(), ptrs.data(), nl, s);
    g.tile_lo = static_cast<int>(mt_begin[lo[w]]);
    g.tile_cap = static_cast<int>(mt_begin[hi[w]] - mt_begin[lo[w]]);
    if (st == MOE_OK && err == hipSuccess)
      err = launch_routed(sh, x, t0, g, row_tok, row_slot, h, y, s);
    // The wave's table entries go back to NULL: a tile outside the planned waves (only
    // possible with caller counts that differ from the chunk's own) then finds no line and
    // writes NaN, instead of reading a line a later copy may be refilling.
    if (st == MOE_OK && err == hipSuccess) {
      std::vector<const void*> none(nl, nullptr);
      err = launch_upload_pairs(wtab, wexp[w].data(), none.data(), nl, s);
    }
    if (st == MOE_OK && err != hipSuccess)
      st = set_error(MOE_ERR_HIP, "wave %d launch: %s", w, hipGetErrorString(err));
    moe_status rst = ring_release(R, wlines[w].data(), nl, s);
    if (st == MOE_OK) st = rst;
    if (st != MOE_OK) { release_held(i + 1); return st; }
    R->stats.waves++;
  }
  return MOE_OK;
}

// A layer call's deferred shared down + combine: a chunk on 256-, 128- or 64-row routed tiles
// leaves its shared down GEMM and combine to the next chunk's gate/up launch
// (launch_gu_mixed_combine). The deferring chunks alternate between two h_shared blocks, since
// a chunk's gate/up writes its own while the previous chunk's down GEMM reads that one; every
// chunk of the call uses the workspace layout of layout_rows rows, so Y, which the next
// chunk's routed down GEMM overwrites only after that launch, is at one place.
struct DeferredCombine {
  void* h_shared[2] = {nullptr, nullptr};
  int next = 0;                 // block of the next deferring chunk
  bool pending = false;         // a chunk's shared down + combine has not run yet
  const void* hs = nullptr;     // that chunk's h_shared block, first row and rows
  int64_t t0 = 0, n = 0;
  int64_t layout_rows = 0;
};

// Runs the pending shared down + combine in a launch of its own (after the last chunk, or
// before a chunk whose tiles cannot take it). y: the workspace's Y, still that chunk's.
hipError_t flush_deferred(const moe_layer* L, DeferredCombine* dc, const float* y,
                          const float* weights, void* out, hipStream_t s) {
  if (!dc->pending) return hipSuccess;
  dc->pending = false;
  const moe_shape& sh = L->shape;
  return launch_down_combine(sh.dtype, dc->hs, dc->n, sh.d, sh.inter_shared, L->w_down_shared,
                             y, weights, dc->t0, sh.top_k, out, s);
}

moe_status chunk_impl(const moe_layer* L, bool offloaded, const void* x, const int32_t* ids,
                      const float* weights, int64_t t0, int64_t n, const int32_t* counts_host,
                      void* out, void* ws_v, size_t ws_bytes, hipStream_t s, hipStream_t cs,
                      const Pinned* pin = nullptr, int32_t* counts_out = nullptr,
                      const WsLayout* lists = nullptr, DeferredCombine* defer = nullptr) {
  const moe_shape& sh = L->shape;
  const int E = sh.n_experts, k = sh.top_k;
  WsLayout W;
  ws_layout(sh, defer ? defer->layout_rows : n, &W);
  if (ws_bytes < W.total)
    return set_error(MOE_ERR_WORKSPACE, "workspace %zu bytes, %zu needed for %lld rows",
                     ws_bytes, W.total, static_cast<long long>(n));
  char* ws = static_cast<char*>(ws_v);
  if (lists) {                  // the chunk was bucketed up front (moe_prefill_layer)
    W.blk_counts = lists->blk_counts;
    W.blk_base = lists->blk_base;
    W.counts = lists->counts;
    W.offsets = lists->offsets;
    W.meta = lists->meta;
    W.mtiles = lists->mtiles;
    W.row_tok = lists->row_tok;
    W.row_slot = lists->row_slot;
  }
  const void** wtab = reinterpret_cast<const void**>(ws + W.wtab);
  // The shared expert's GU depends only on x. With every expert resident it runs in order
  // on the caller's stream: its GEMM and the routed ones each fill the chip, and running them
  // side by side measured slower than in sequence. With a ring it runs on a side stream
  // (joined before the last kernel), filling the time the routed GEMMs wait for copies. Its
  // down GEMM runs last, with the combine folded into its epilogue (in a layer call, possibly
  // inside the next chunk's gate/up launch: DeferredCombine).
  SideStream side;
  JoinOnExit pending{side, s};
  hipStream_t ss = offloaded ? nullptr : s;
  const int bm = routed_tile_rows(n, k, E);
  // With every expert resident, the shared GU's units join the routed GU's launch
  // (launch_gu_mixed, on the routed tile shape), so the compute-bound shared tiles run beside
  // the weight-streaming routed ones. A chunk on decode tiles of at most kMixedDecodeRows tokens
  // does the same with both shared GEMMs (16-row blocks): alone, each would fill a few dozen CUs
  // and wait on load latency. Its shared down GEMM then writes S to the workspace and the stand-alone
  // combine follows (the same operations in the same order as the folded one, the same bits).
  // (MOE_OPT_FUSED_GU_DOWN, where it applies, keeps the routed GEMMs in its fused launch.)
  const bool fused = g_opt_fused_gu_down.load(std::memory_order_relaxed) &&
                     gu_down_fused_supported(sh.dtype, bm, sh.inter);
  const bool mixed = !offloaded && sh.inter_shared && !fused && gu_mixed_supported(bm, n);
  const bool small = mixed && bm == kDecodeTileRows;
  // In a layer call, a chunk on tiles gu_mixed_combine_supported takes leaves its shared down +
  // combine to the next chunk's gate/up launch (DeferredCombine); on decode tiles (193 to 512
  // tokens) its shared gate/up runs in that launch too.
  const bool defer_this = defer && !offloaded && sh.inter_shared && !fused && !small &&
                          gu_mixed_combine_supported(bm, n);
  float* y = reinterpret_cast<float*>(ws + W.y);
  if (defer && !defer_this) MOE_HIP(flush_deferred(L, defer, y, weights, out, s));
  if (sh.inter_shared && !mixed && !defer_this) {
    if (offloaded) {
      MOE_HIP(side.fork(s));
      ss = side.stream;
    }
    MOE_HIP(launch_gu_dense(sh.dtype, x, t0, n, sh.d, sh.inter_shared, L->w_gu_shared,
                            ws + W.h_shared, ss));
    if (offloaded) {
      MOE_HIP(side.record_done());
      pending.armed = true;
    }
  }
  // Resident lines at a uniform stride (one block of E lines) need no table; otherwise the
  // table is uploaded to the workspace (offloaded entries are filled per wave).
  int64_t stride = 0;
  const bool uniform = !offloaded && uniform_lines(L->expert_lines, E, &stride);
  if (!uniform) MOE_HIP(launch_upload_ptrs(wtab, L->expert_lines, 0, E, s));
  if (!lists) MOE_HIP(launch_bucket(ids + t0 * k, n, k, E, bm, ws, W, s, counts_out));
  if (!offloaded) {
    GemmGroups g{reinterpret_cast<const MTile*>(ws + W.mtiles),
                 reinterpret_cast<const int32_t*>(ws + W.meta) + kMetaMTiles,
                 reinterpret_cast<const int32_t*>(ws + W.offsets),
                 reinterpret_cast<const int32_t*>(ws + W.counts), wtab,
                 uniform ? static_cast<const char*>(L->expert_lines[0]) : nullptr, stride, 0,
                 static_cast<int>(n * k / bm + std::min<int64_t>(E, n * k)), bm};
    const int32_t* row_tok = reinterpret_cast<const int32_t*>(ws + W.row_tok);
    const int32_t* row_slot = reinterpret_cast<const int32_t*>(ws + W.row_slot);
    if (small) {
      float* s_small = reinterpret_cast<float*>(ws + W.s_small);
      MOE_HIP(launch_gu_mixed(sh.dtype, x, t0, n, sh.d, sh.inter, sh.inter_shared,
                              L->w_gu_shared, ws + W.h_shared, g, row_tok, ws + W.h, s));
      MOE_HIP(launch_down_mixed(sh.dtype, ws + W.h_shared, n, sh.d, sh.inter_shared,
                                L->w_down_shared, s_small, ws + W.h, sh.inter, g, row_slot, y,
                                s));
      MOE_HIP(launch_combine(sh.dtype, y, s_small, weights, t0, n, k, sh.d, out, s));
      return MOE_OK;
    }
    if (defer_this) {
      void* hs = defer->h_shared[defer->next];
      MOE_HIP(launch_gu_mixed_combine(sh.dtype, x, t0, n, sh.d, sh.inter, sh.inter_shared,
                                      L->w_gu_shared, hs, g, row_tok, ws + W.h, defer->hs,
                                      defer->t0, defer->pending ? defer->n : 0,
                                      L->w_down_shared, y, weights, k, out, s));
      MOE_HIP(launch_down_routed(sh.dtype, ws + W.h, sh.d, sh.inter, g, row_slot, y, s));
      defer->pending = true;
      defer->hs = hs;
      defer->t0 = t0;
      defer->n = n;
      defer->next ^= 1;
      return MOE_OK;
    }
    if (mixed) {
      MOE_HIP(launch_gu_mixed(sh.dtype, x, t0, n, sh.d, sh.inter, sh.inter_shared,
                              L->w_gu_shared, ws + W.h_shared, g, row_tok, ws + W.h, s));
      MOE_HIP(launch_down_routed(sh.dtype, ws + W.h, sh.d, sh.inter, g, row_slot, y, s));
    } else {
      MOE_HIP(launch_routed(sh, x, t0, g, row_tok, row_slot, ws + W.h, y, s));
    }
  } else {
    moe_status st = ring_waves(L, x, t0, n, counts_host, ws, W, s, cs ? cs : s, pin);
    // Join even on failure, so the caller's stream never runs ahead of the side work.
    if (pending.armed) MOE_HIP(pending.join());
    if (st != MOE_OK) return st;
  }
  if (sh.inter_shared)
    MOE_HIP(launch_down_combine(sh.dtype, ws + W.h_shared, n, sh.d, sh.inter_shared,
                                L->w_down_shared, y, weights, t0, k, out, s));
  else
    MOE_HIP(launch_combine(sh.dtype, y, nullptr, weights, t0, n, k, sh.d, out, s));
  return MOE_OK;
}

moe_status check_rows(int64_t T, const moe_shape& sh) {
  if (T < 0) return set_error(MOE_ERR_INVALID, "T=%lld", static_cast<long long>(T));
  if (T > (int64_t{1} << 31) / sh.top_k - 1)
    return set_error(MOE_ERR_INVALID, "T=%lld too large (T*k must fit int32)",
                     static_cast<long long>(T));
  return MOE_OK;
}

}  // namespace

moe_status prefill_chunk_checked(const moe_layer* layer, const void* x, const int32_t* ids,
                                 const float* weights, int64_t T, int64_t t0, int64_t n,
                                 const int32_t* counts_host, void* out, void* ws,
                                 size_t ws_bytes, void* stream, void* copy_stream,
                                 bool resident_only, void* (*ws_of_device)(moe_status*)) {
  moe_status st = check_layer(layer);
  if (st != MOE_OK) return st;
  if ((st = check_rows(T, layer->shape)) != MOE_OK) return st;
  if (t0 < 0 || n < 0 || t0 + n > T)
    return set_error(MOE_ERR_INVALID, "rows [%lld, %lld) outside [0, %lld)",
                     static_cast<long long>(t0), static_cast<long long>(t0 + n),
                     static_cast<long long>(T));
  bool offloaded = false;
  if ((st = check_experts(layer, &offloaded)) != MOE_OK) return st;
  if (offloaded && resident_only)
    return set_error(MOE_ERR_UNSUPPORTED, "this entry point takes resident experts only");
  if (ws_of_device) {                 // the workspace is the library's own array on this device
    WsLayout W;
    ws_layout(layer->shape, n, &W);
    if (W.total > ws_bytes)
      return set_error(MOE_ERR_WORKSPACE, "%lld rows need %zu bytes of workspace, %zu available",
                       static_cast<long long>(n), W.total, ws_bytes);
  }
  if (n == 0) return MOE_OK;
  if (ws_of_device && !(ws = ws_of_device(&st))) return st;
  if (!x || !ids || !weights || !out || !ws)
    return set_error(MOE_ERR_INVALID, "NULL tensor argument");
  if (!aligned(x, 16) || !aligned(out, 16) || !aligned(ids, 4) || !aligned(weights, 4) ||
      !aligned(ws, 256))
    return set_error(MOE_ERR_INVALID, "misaligned tensor argument (ws needs 256 bytes)");
  return chunk_impl(layer, offloaded, x, ids, weights, t0, n, counts_host, out, ws, ws_bytes,
                    static_cast<hipStream_t>(stream), static_cast<hipStream_t>(copy_stream));
}

bool ws_layout(const moe_shape& sh, int64_t max_n, WsLayout* L) {
  if (max_n < 1) max_n = 1;
  const int64_t E = sh.n_experts, k = sh.top_k, d = sh.d, I = sh.inter, Is = sh.inter_shared;
  const size_t elt = elt_bytes(sh.dtype);
  const int64_t rows = max_n * k;
  const int64_t nb = (max_n + kTokBlock - 1) / kTokBlock;
  const int64_t max_mt = rows / kMinTileRows + std::min<int64_t>(E, rows);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align_up(bytes);
    return o;
  };
  L->wtab = take(sizeof(void*) * E);
  L->blk_counts = take(sizeof(int32_t) * nb * E);
  L->blk_base = take(sizeof(int32_t) * nb * E);
  L->counts = take(sizeof(int32_t) * E);
  L->offsets = take(sizeof(int32_t) * (E + 1));
  L->meta = take(sizeof(int32_t) * kMetaWords);
  L->mtiles = take(sizeof(MTile) * max_mt);
  L->row_tok = take(sizeof(int32_t) * rows);
  L->row_slot = take(sizeof(int32_t) * rows);
  L->h = take(elt * rows * I);
  L->h_shared = take(elt * max_n * Is);
  L->y = take(sizeof(float) * rows * d);
  L->s_small = take(Is ? sizeof(float) * std::min<int64_t>(max_n, kMixedDecodeRows) * d : 0);
  L->total = off;
  L->max_n = max_n;
  L->max_rows = rows;
  L->max_mtiles = max_mt;
  L->n_blocks = nb;
  return true;
}

// Workspace of a layer call of two or more chunks of `chunk` tokens that buckets them all up
// front: the one-chunk layout for `chunk` rows (base bytes), then every chunk's member lists
// in turn (that layout's block histograms through row_slot, one contiguous block of
// list_stride bytes per chunk), then a second h_shared block (none without a shared expert)
// for the deferred shared down + combine. `lists` is the one-chunk layout with its list
// offsets moved to chunk 0's block.
struct LayerWs {
  WsLayout lists;
  size_t base, list_stride, h_shared2, total;
};

void layer_ws_layout(const moe_shape& sh, int64_t T, int64_t chunk, LayerWs* L) {
  WsLayout& W = L->lists;
  ws_layout(sh, chunk, &W);
  L->base = W.total;
  L->list_stride = W.h - W.blk_counts;
  const size_t shift = L->base - W.blk_counts;
  W.blk_counts += shift;
  W.blk_base += shift;
  W.counts += shift;
  W.offsets += shift;
  W.meta += shift;
  W.mtiles += shift;
  W.row_tok += shift;
  W.row_slot += shift;
  const int64_t n_chunks = (T + chunk - 1) / chunk;
  L->h_shared2 = L->base + static_cast<size_t>(n_chunks) * L->list_stride;
  L->total = L->h_shared2 + (W.y - W.h_shared);
}

}  // namespace moe

using moe::set_error;

extern "C" {

int32_t moe_abi_version(void) { return MOE_ABI_VERSION; }

moe_status moe_set_option(int32_t option, int32_t value) {
  moe::clear_error();
  if (option != MOE_OPT_FUSED_GU_DOWN)
    return moe::set_error(MOE_ERR_INVALID, "unknown option %d", option);
  moe::g_opt_fused_gu_down.store(value != 0 ? 1 : 0, std::memory_order_relaxed);
  return MOE_OK;
}

moe_status moe_get_option(int32_t option, int32_t* value) {
  moe::clear_error();
  if (!value) return moe::set_error(MOE_ERR_INVALID, "value is NULL");
  if (option != MOE_OPT_FUSED_GU_DOWN)
    return moe::set_error(MOE_ERR_INVALID, "unknown option %d", option);
  *value = moe::g_opt_fused_gu_down.load(std::memory_order_relaxed);
  return MOE_OK;
}

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID: return "MOE_ERR_INVALID";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_RING: return "MOE_ERR_RING";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
  }
  return "MOE_ERR_UNKNOWN";
}

const char* moe_last_error(void) { return moe::last_error_text(); }

size_t moe_workspace_bytes(const moe_shape* shape, int64_t max_chunk_tokens) {
  if (moe::check_shape(shape) != MOE_OK || max_chunk_tokens < 0) return 0;
  if (max_chunk_tokens > (int64_t{1} << 31) / shape->top_k - 1) return 0;
  moe::WsLayout L;
  moe::ws_layout(*shape, max_chunk_tokens, &L);
  return L.total;
}

size_t moe_layer_workspace_bytes(const moe_shape* shape, int64_t T, int64_t chunk) {
  if (chunk < 1 || T < 0) return 0;
  const size_t base = moe_workspace_bytes(shape, std::min(chunk, std::max<int64_t>(T, 1)));
  if (base == 0) return 0;
  const int64_t n_chunks = (T + chunk - 1) / chunk;
  if (n_chunks < 2) return base;
  moe::LayerWs L;
  moe::layer_ws_layout(*shape, T, chunk, &L);
  return L.total;
}

moe_status moe_workspace_offsets(const moe_shape* shape, int64_t n, moe_ws_offsets* out) {
  moe::clear_error();
  moe_status st = moe::check_shape(shape);
  if (st != MOE_OK) return st;
  if (!out || n < 0 || n > (int64_t{1} << 31) / shape->top_k - 1)
    return set_error(MOE_ERR_INVALID, "bad arguments");
  moe::WsLayout L;
  moe::ws_layout(*shape, n, &L);
  out->counts = L.counts;
  out->offsets = L.offsets;
  out->row_tok = L.row_tok;
  out->row_slot = L.row_slot;
  out->h = L.h;
  out->h_shared = L.h_shared;
  out->y = L.y;
  out->total = L.total;
  return MOE_OK;
}

moe_status moe_prefill_route(const moe_layer* layer, const void* x, int64_t T, int64_t chunk,
                             int32_t* ids, float* weights, int32_t* chunk_counts, float* logits,
                             void* stream) {
  moe::clear_error();
  moe_status st = moe::check_layer(layer);
  if (st != MOE_OK) return st;
  if ((st = moe::check_rows(T, layer->shape)) != MOE_OK) return st;
  if (chunk < 1) return set_error(MOE_ERR_INVALID, "chunk=%lld", static_cast<long long>(chunk));
  if (T == 0) return MOE_OK;
  if (!x || !ids || !weights || !chunk_counts || !logits)
    return set_error(MOE_ERR_INVALID, "NULL tensor argument");
  if (!moe::aligned(x, 16) || !moe::aligned(ids, 4) || !moe::aligned(weights, 4) ||
      !moe::aligned(chunk_counts, 4) || !moe::aligned(logits, 4))
    return set_error(MOE_ERR_INVALID, "misaligned tensor argument");
  return moe::route_impl(layer, x, T, chunk, ids, weights, chunk_counts, logits,
                         static_cast<hipStream_t>(stream));
}

moe_status moe_prefill_chunk(const moe_layer* layer, const void* x, const int32_t* ids,
                             const float* weights, int64_t T, int64_t t0, int64_t n,
                             const int32_t* counts_host, void* out, void* ws, size_t ws_bytes,
                             void* stream, void* copy_stream) {
  moe::clear_error();
  return moe::prefill_chunk_checked(layer, x, ids, weights, T, t0, n, counts_host, out, ws,
                                    ws_bytes, stream, copy_stream, /*resident_only=*/false,
                                    nullptr);
}

moe_status moe_prefill_layer(const moe_layer* layer, const void* x, int64_t T, int64_t chunk,
                             int32_t* ids, float* weights, int32_t* chunk_counts, float* logits,
                             void* out, void* ws, size_t ws_bytes, void* stream,
                             void* copy_stream) {
  moe::clear_error();
  moe_status st = moe::check_layer(layer);
  if (st != MOE_OK) return st;
  if ((st = moe::check_rows(T, layer->shape)) != MOE_OK) return st;
  if (chunk < 1) return set_error(MOE_ERR_INVALID, "chunk=%lld", static_cast<long long>(chunk));
  bool offloaded = false;
  if ((st = moe::check_experts(layer, &offloaded)) != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!x || !ids || !weights || !chunk_counts || !logits || !out || !ws)
    return set_error(MOE_ERR_INVALID, "NULL tensor argument");
  if (!moe::aligned(x, 16) || !moe::aligned(out, 16) || !moe::aligned(ids, 4) ||
      !moe::aligned(weights, 4) || !moe::aligned(chunk_counts, 4) ||
      !moe::aligned(logits, 4) || !moe::aligned(ws, 256))
    return set_error(MOE_ERR_INVALID, "misaligned tensor argument (ws needs 256 bytes)");
  const int64_t cmax = std::min(chunk, T);
  const size_t need = moe_workspace_bytes(&layer->shape, cmax);
  if (ws_bytes < need)
    return set_error(MOE_ERR_WORKSPACE, "workspace %zu bytes, %zu needed for chunk %lld",
                     ws_bytes, need, static_cast<long long>(cmax));
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipStream_t cs = static_cast<hipStream_t>(copy_stream);
  // With every expert resident nothing reads the chunk counts before the chunks run, so
  // each chunk's bucketing writes its own row (the same integers: ids from the router never
  // repeat an expert within a token) and the per-chunk histogram launch is saved; a ring
  // plans its waves from them, so they are counted up front.
  if ((st = moe::route_impl(layer, x, T, chunk, ids, weights, chunk_counts, logits, s,
                            /*counts_in_chunks=*/!offloaded)) != MOE_OK)
    return st;
  const int E = layer->shape.n_experts;
  const int64_t n_chunks = (T + chunk - 1) / chunk;
  std::vector<int32_t> hc;
  if (offloaded) {             // one device-to-host copy of every chunk's expert counts
    hc.resize(static_cast<size_t>(n_chunks) * E);
    hipError_t err = hipMemcpyAsync(hc.data(), chunk_counts, hc.size() * sizeof(int32_t),
                                    hipMemcpyDeviceToHost, s);
    if (err == hipSuccess) err = hipStreamSynchronize(s);
    if (err != hipSuccess)
      return set_error(MOE_ERR_HIP, "chunk counts to host: %s", hipGetErrorString(err));
  }
  // With a ring and several chunks, the experts most chunks use stay in held lines for the
  // whole call (staged up front, released after the last chunk).
  moe::Pinned pin;
  if (offloaded && n_chunks >= 2) {
    pin.experts = moe::choose_pinned(layer, hc.data(), n_chunks);
    if (!pin.experts.empty()) {
      bool all_offloaded = true;
      for (int e = 0; e < E; ++e) all_offloaded &= layer->expert_lines[e] == nullptr;
      pin.lines.resize(pin.experts.size());
      st = moe::ring_stage(layer->ring, layer->layer_id, pin.experts.data(),
                           static_cast<int32_t>(pin.experts.size()), cs ? cs : s,
                           pin.lines.data(), nullptr, /*two_streams=*/true, MOE_COPY_INITIAL,
                           /*hold=*/true, all_offloaded);
      if (st == MOE_ERR_RING) {   // lines held elsewhere (public staging calls): no pinning
        moe::clear_error();
        pin.experts.clear();
        pin.lines.clear();
        st = MOE_OK;
      }
      if (st != MOE_OK) return st;
    }
  }
  // With every expert resident and room for every chunk's member lists, all chunks are
  // bucketed up front in one set of launches (the same kernels on the same ids, so the same
  // lists), and no chunk's GEMMs wait for bucketing launches of their own. With a shared
  // expert, chunks then also defer their shared down + combine to the next chunk's gate/up
  // launch where the tiles allow (DeferredCombine); the bytes are the same.
  moe::LayerWs lw{};
  const bool prebucket = !offloaded && n_chunks >= 2 &&
                         ws_bytes >= moe_layer_workspace_bytes(&layer->shape, T, chunk);
  moe::DeferredCombine dc;
  moe::DeferredCombine* defer = nullptr;
  if (prebucket) {
    const int k = layer->shape.top_k;
    moe::layer_ws_layout(layer->shape, T, chunk, &lw);
    hipError_t err = moe::launch_bucket_chunks(
        ids, T, chunk, k, E, moe::routed_tile_rows(chunk, k, E),
        moe::routed_tile_rows(T - (n_chunks - 1) * chunk, k, E), static_cast<char*>(ws),
        lw.lists, static_cast<int64_t>(lw.list_stride), chunk_counts, s);
    if (err != hipSuccess)
      return set_error(MOE_ERR_HIP, "bucketing: %s", hipGetErrorString(err));
    if (layer->shape.inter_shared > 0) {
      dc.h_shared[0] = static_cast<char*>(ws) + lw.lists.h_shared;
      dc.h_shared[1] = static_cast<char*>(ws) + lw.h_shared2;
      dc.layout_rows = chunk;
      defer = &dc;
    }
  }
  for (int64_t c = 0; c < n_chunks; ++c) {
    const int64_t t0 = c * chunk;
    const int64_t n = std::min(chunk, T - t0);
    moe::WsLayout lc = lw.lists;
    if (prebucket) {
      const size_t o = static_cast<size_t>(c) * lw.list_stride;
      lc.blk_counts += o;
      lc.blk_base += o;
      lc.counts += o;
      lc.offsets += o;
      lc.meta += o;
      lc.mtiles += o;
      lc.row_tok += o;
      lc.row_slot += o;
    }
    st = moe::chunk_impl(layer, offloaded, x, ids, weights, t0, n,
                         offloaded ? hc.data() + c * E : nullptr, out, ws, ws_bytes, s, cs,
                         pin.experts.empty() ? nullptr : &pin,
                         offloaded || prebucket ? nullptr : chunk_counts + c * E,
                         prebucket ? &lc : nullptr, defer);
    if (st != MOE_OK) break;
  }
  if (st == MOE_OK && defer) {
    hipError_t err = moe::flush_deferred(
        layer, defer, reinterpret_cast<const float*>(static_cast<char*>(ws) + lw.lists.y),
        weights, out, s);
    if (err != hipSuccess)
      st = set_error(MOE_ERR_HIP, "shared down + combine: %s", hipGetErrorString(err));
  }
  if (!pin.experts.empty()) {
    moe_status rst = moe::ring_release(layer->ring, pin.lines.data(),
                                       static_cast<int32_t>(pin.lines.size()), s);
    if (st == MOE_OK) st = rst;
  }
  return st;
}

moe_status moe_add_rmsnorm(const void* x, const void* delta, int64_t T, int32_t d,
                           int32_t dtype, float eps, void* x_out, void* normed, void* stream) {
  moe::clear_error();
  if (T < 0 || d < 1 || d > (1 << 20)) return set_error(MOE_ERR_INVALID, "T or d out of range");
  if (dtype != MOE_BF16 && dtype != MOE_F32) return set_error(MOE_ERR_INVALID, "dtype");
  if (!(eps >= 0.0f)) return set_error(MOE_ERR_INVALID, "eps must be >= 0");
  if (T == 0) return MOE_OK;
  if (!x || !normed || (delta && !x_out))
    return set_error(MOE_ERR_INVALID, "NULL tensor argument");
  MOE_HIP(moe::launch_add_rmsnorm(dtype, x, delta, T, d, eps, x_out, normed,
                                  static_cast<hipStream_t>(stream)));
  return MOE_OK;
}

}  // extern "C"
