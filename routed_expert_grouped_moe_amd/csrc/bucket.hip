// Bucketing of one chunk's token-slots by expert, on the GPU: per-block histogram, one scan
// kernel (block bases, expert offsets, M-tile list) and a stable permute. The pages build
// these per-expert member lists on the CPU ("EXL3 on upstream", PR #1113, "Latest prefill
// efficiency candidate"); here they never leave the device, so the resident path needs no
// host synchronisation.
//
// Row order inside an expert is token order (a stable permute), so the member list of each
// expert is unique and the whole bucketing is reproducible bit for bit.
//
// Slots whose id is outside [0, E), or repeats an expert already listed for the same token,
// are dropped by every kernel here alike (a token's slots are taken in order, so the first
// occurrence counts): counts, offsets and member lists then describe exactly the slots kept,
// every member-list row is written, and no access depends on an unchecked id. Ids as
// moe_prefill_route writes them are always kept.
#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "moe_internal.h"
#include "profile.h"

namespace moe {
namespace {

constexpr int kMaxE = 1024;

// Marks token `tid` of the block in expert e's 256-bit LDS mask; true if the slot is kept (e in
// range and not yet marked for this token).
__device__ __forceinline__ bool mark_slot(uint32_t* mask, int e, int E, int tid) {
  if (static_cast<unsigned>(e) >= static_cast<unsigned>(E)) return false;
  const uint32_t bit = 1u << (tid & 31);
  return (atomicOr(&mask[e * (kTokBlock / 32) + (tid >> 5)], bit) & bit) == 0u;
}

// Whether slot j (expert e) of a token is kept: e in range and no earlier slot of the token
// names e. Slots below 64 use the bits mark_slot returned; later ones (k > 64) are checked
// against the token's earlier ids.
__device__ __forceinline__ bool slot_kept(const int32_t* tok_ids, int j, int e, int E,
                                          uint64_t kept) {
  if (j < 64) return (kept >> j) & 1u;
  if (static_cast<unsigned>(e) >= static_cast<unsigned>(E)) return false;
  for (int i = 0; i < j; ++i)
    if (tok_ids[i] == e) return false;
  return true;
}

// Which chunk a workgroup buckets: chunk blockIdx.y of a prompt of T tokens cut into chunks of
// `chunk`, its lists in the block of workspace stride * blockIdx.y bytes past the pointers
// given (one chunk: chunk = T = n, stride 0). The bucketing of every chunk of a layer call can
// so run in one set of launches, each chunk's lists exactly those of its own launches.
struct ChunkSeg {
  int64_t chunk, T;
  int64_t stride;        // bytes between consecutive chunks' list blocks
  int bm_last;           // M-tile rows of the last chunk (the others: the bm argument)
  int32_t* counts_out;   // [chunks, E] each chunk's expert counts as well, or NULL
};
__device__ __forceinline__ int64_t seg_t0(const ChunkSeg& s) {
  return static_cast<int64_t>(blockIdx.y) * s.chunk;
}
__device__ __forceinline__ int64_t seg_n(const ChunkSeg& s) {
  return min(s.chunk, s.T - seg_t0(s));
}
template <typename P>
__device__ __forceinline__ P* seg_at(P* p, const ChunkSeg& s) {
  typedef typename std::conditional<std::is_const<P>::value, const char, char>::type C;
  return reinterpret_cast<P*>(reinterpret_cast<C*>(p) + static_cast<int64_t>(blockIdx.y) * s.stride);
}
__device__ __forceinline__ int seg_bm(const ChunkSeg& s, int bm) {
  return static_cast<int64_t>(blockIdx.y) == (s.T - 1) / s.chunk ? s.bm_last : bm;
}
__device__ __forceinline__ int32_t* seg_counts_out(const ChunkSeg& s, int E) {
  return s.counts_out ? s.counts_out + static_cast<int64_t>(blockIdx.y) * E : nullptr;
}

// blk_counts[b][e] = kept slots of tokens [b*256, b*256+256) routed to e (LDS histogram).
__global__ __launch_bounds__(kTokBlock) void block_hist_kernel(const int32_t* __restrict__ ids,
                                                               int k, int E,
                                                               int32_t* __restrict__ blk_counts,
                                                               ChunkSeg seg) {
  __shared__ int32_t hist[kMaxE];
  __shared__ uint32_t mask[kMaxE * (kTokBlock / 32)];
  const int64_t n = seg_n(seg);
  if (static_cast<int64_t>(blockIdx.x) * kTokBlock >= n) return;   // past this chunk's blocks
  ids += seg_t0(seg) * k;
  blk_counts = seg_at(blk_counts, seg);
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += kTokBlock) hist[e] = 0;
  for (int w = tid; w < E * (kTokBlock / 32); w += kTokBlock) mask[w] = 0u;
  __syncthreads();
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kTokBlock + tid;
  if (t < n)
    for (int j = 0; j < k; ++j) {
      const int e = ids[t * k + j];
      if (mark_slot(mask, e, E, tid)) atomicAdd(&hist[e], 1);
    }
  __syncthreads();
  int32_t* out = blk_counts + static_cast<int64_t>(blockIdx.x) * E;
  for (int e = tid; e < E; e += kTokBlock) out[e] = hist[e];
}

// One workgroup of 1024 threads; thread e owns expert e.
//   blk_base[b][e] = slots of e in blocks before b; counts[e]; offsets = exclusive scan of
//   counts; M-tiles: expert e contributes ceil(counts[e]/bm) tiles (e, 0), (e, bm), ... at
//   position (exclusive scan of the tile counts); meta = {number of tiles, number of rows};
//   counts_out (if not NULL) = counts as well, the chunk's row of the layer call's
//   chunk_counts.
__global__ __launch_bounds__(1024) void scan_kernel(const int32_t* __restrict__ blk_counts,
                                                    int E, int bm,
                                                    int32_t* __restrict__ blk_base,
                                                    int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ offsets,
                                                    MTile* __restrict__ mtiles,
                                                    int32_t* __restrict__ meta, ChunkSeg seg) {
  __shared__ int32_t s_rows[kMaxE];
  __shared__ int32_t s_tiles[kMaxE];
  const int nb = static_cast<int>((seg_n(seg) + kTokBlock - 1) / kTokBlock);
  blk_counts = seg_at(blk_counts, seg);
  blk_base = seg_at(blk_base, seg);
  counts = seg_at(counts, seg);
  offsets = seg_at(offsets, seg);
  mtiles = seg_at(mtiles, seg);
  meta = seg_at(meta, seg);
  int32_t* counts_out = seg_counts_out(seg, E);
  bm = seg_bm(seg, bm);
  const int e = threadIdx.x;
  int32_t run = 0;
  if (e < E) {
    constexpr int kBatch = 16;           // loads of a batch are issued before their sums
    for (int b0 = 0; b0 < nb; b0 += kBatch) {
      int32_t c[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j)
        c[j] = b0 + j < nb ? blk_counts[static_cast<int64_t>(b0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < kBatch; ++j)
        if (b0 + j < nb) {
          blk_base[static_cast<int64_t>(b0 + j) * E + e] = run;
          run += c[j];
        }
    }
    counts[e] = run;
    if (counts_out) counts_out[e] = run;
  }
  const int32_t ntile = (run + bm - 1) / bm;
  s_rows[e] = run;
  s_tiles[e] = ntile;
  __syncthreads();
  for (int off = 1; off < kMaxE; off <<= 1) {    // inclusive Hillis-Steele scans
    const int32_t a = e >= off ? s_rows[e - off] : 0;
    const int32_t b = e >= off ? s_tiles[e - off] : 0;
    __syncthreads();
    s_rows[e] += a;
    s_tiles[e] += b;
    __syncthreads();
  }
  const int32_t row_off = s_rows[e] - run;
  const int32_t tile_off = s_tiles[e] - ntile;
  if (e < E) {
    offsets[e] = row_off;
    for (int i = 0; i < ntile; ++i) mtiles[tile_off + i] = MTile{e, i * bm};
  }
  if (e == kMaxE - 1) {
    offsets[E] = s_rows[e];
    meta[kMetaMTiles] = s_tiles[e];
    meta[kMetaRows] = s_rows[e];
  }
}

// Stable permute. Block b (tokens [b*256, b*256+256)) marks, per expert, which of its tokens
// chose that expert in a 256-bit LDS mask; a token's rank among the block's tokens of expert
// e is the number of marked tokens before it. Row = offsets[e] + blk_base[b][e] + rank.
__global__ __launch_bounds__(kTokBlock) void permute_kernel(const int32_t* __restrict__ ids,
                                                            int k, int E,
                                                            const int32_t* __restrict__ blk_base,
                                                            const int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ row_tok,
                                                            int32_t* __restrict__ row_slot,
                                                            ChunkSeg seg) {
  __shared__ uint32_t mask[kMaxE * (kTokBlock / 32)];
  const int64_t n = seg_n(seg);
  if (static_cast<int64_t>(blockIdx.x) * kTokBlock >= n) return;   // past this chunk's blocks
  ids += seg_t0(seg) * k;
  blk_base = seg_at(blk_base, seg);
  offsets = seg_at(offsets, seg);
  row_tok = seg_at(row_tok, seg);
  row_slot = seg_at(row_slot, seg);
  const int tid = threadIdx.x;
  for (int w = tid; w < E * (kTokBlock / 32); w += kTokBlock) mask[w] = 0u;
  __syncthreads();
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kTokBlock + tid;
  const bool valid = t < n;
  const int word = tid >> 5;
  const uint32_t bit = 1u << (tid & 31);
  uint64_t kept = 0;              // slots j < 64 kept (k > 64: later slots are re-checked)
  if (valid)
    for (int j = 0; j < k; ++j)
      if (mark_slot(mask, ids[t * k + j], E, tid) && j < 64) kept |= uint64_t{1} << j;
  __syncthreads();
  if (!valid) return;
  const int32_t* base = blk_base + static_cast<int64_t>(blockIdx.x) * E;
  for (int j = 0; j < k; ++j) {
    const int e = ids[t * k + j];
    if (!slot_kept(ids + t * k, j, e, E, kept)) continue;
    const uint32_t* m = mask + e * (kTokBlock / 32);
    int rank = __popc(m[word] & (bit - 1u));
    for (int w = 0; w < word; ++w) rank += __popc(m[w]);
    const int64_t r = static_cast<int64_t>(offsets[e]) + base[e] + rank;
    row_tok[r] = static_cast<int32_t>(t);
    row_slot[r] = static_cast<int32_t>(t * k + j);
  }
}

// Permute with the scan folded in, for chunks of at most kScanBlocks token blocks: every block
// sums the block histograms itself (its own prefix over earlier blocks and the totals over all
// nb), scans the totals in LDS and places its tokens as permute_kernel does; block 0 also
// writes counts, offsets, the M-tile list and meta exactly as scan_kernel does. One launch per
// chunk fewer; the integers are the same.
// (at 16 blocks the serial sums over the block histograms cost more than the launch they save:
// 85 against 79 us per layer at 4,096-token chunks; at 8 and 4 blocks 124 against 152 and 214
// against 303 us)
// kOneBlock: a chunk of one token block counts its experts from its own LDS masks (the
// popcount of expert e's mask is the block's rows of e), so it needs no histogram launch.
constexpr int kScanBlocks = 8;
template <bool kOneBlock>
__global__ __launch_bounds__(kTokBlock) void permute_scan_kernel(
    const int32_t* __restrict__ ids, int k, int E, int bm,
    const int32_t* __restrict__ blk_counts, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, MTile* __restrict__ mtiles, int32_t* __restrict__ meta,
    int32_t* __restrict__ row_tok, int32_t* __restrict__ row_slot, ChunkSeg seg) {
  constexpr int PER = kMaxE / kTokBlock;         // experts per thread in the scans
  __shared__ int32_t s_tot[kMaxE];               // rows of e in the chunk
  __shared__ int32_t s_pre[kMaxE];               // rows of e in blocks before this one
  __shared__ int32_t s_off[kMaxE + 1];           // exclusive scan of s_tot
  __shared__ int32_t s_part[2][kTokBlock];       // per-thread partial sums (rows, tiles)
  __shared__ uint32_t mask[kMaxE * (kTokBlock / 32)];
  const int64_t n = seg_n(seg);
  const int nb = static_cast<int>((n + kTokBlock - 1) / kTokBlock);
  if (static_cast<int>(blockIdx.x) >= nb) return;                   // past this chunk's blocks
  ids += seg_t0(seg) * k;
  blk_counts = seg_at(blk_counts, seg);
  counts = seg_at(counts, seg);
  offsets = seg_at(offsets, seg);
  mtiles = seg_at(mtiles, seg);
  meta = seg_at(meta, seg);
  row_tok = seg_at(row_tok, seg);
  row_slot = seg_at(row_slot, seg);
  int32_t* counts_out = seg_counts_out(seg, E);
  bm = seg_bm(seg, bm);
  const int tid = threadIdx.x, b = blockIdx.x;
  for (int w = tid; w < E * (kTokBlock / 32); w += kTokBlock) mask[w] = 0u;
  const int64_t t = static_cast<int64_t>(b) * kTokBlock + tid;
  const bool valid = t < n;
  const int word = tid >> 5;
  const uint32_t bit = 1u << (tid & 31);
  uint64_t kept = 0;
  auto mark = [&]() {
    if (valid)
      for (int j = 0; j < k; ++j)
        if (mark_slot(mask, ids[t * k + j], E, tid) && j < 64) kept |= uint64_t{1} << j;
  };
  if constexpr (kOneBlock) {
    __syncthreads();
    mark();
    __syncthreads();
  }
  int32_t rows[PER], tiles[PER], rsum = 0, tsum = 0;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int e = tid * PER + q;
    int32_t tot = 0, pre = 0;
    if (kOneBlock && e < E) {
#pragma unroll
      for (int w = 0; w < kTokBlock / 32; ++w) tot += __popc(mask[e * (kTokBlock / 32) + w]);
    } else if (e < E) {
      for (int bb = 0; bb < nb; ++bb) {
        const int32_t c = blk_counts[static_cast<int64_t>(bb) * E + e];
        tot += c;
        if (bb < b) pre += c;
      }
    }
    s_tot[e] = tot;
    s_pre[e] = pre;
    rows[q] = tot;
    tiles[q] = (tot + bm - 1) / bm;
    rsum += rows[q];
    tsum += tiles[q];
  }
  s_part[0][tid] = rsum;
  s_part[1][tid] = tsum;
  __syncthreads();
  for (int off = 1; off < kTokBlock; off <<= 1) {  // inclusive Hillis-Steele scans
    const int32_t a = tid >= off ? s_part[0][tid - off] : 0;
    const int32_t c = tid >= off ? s_part[1][tid - off] : 0;
    __syncthreads();
    s_part[0][tid] += a;
    s_part[1][tid] += c;
    __syncthreads();
  }
  int32_t roff = s_part[0][tid] - rsum, toff = s_part[1][tid] - tsum;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int e = tid * PER + q;
    s_off[e] = roff;
    if (b == 0 && e < E) {
      counts[e] = rows[q];
      if (counts_out) counts_out[e] = rows[q];
      offsets[e] = roff;
      for (int i = 0; i < tiles[q]; ++i) mtiles[toff + i] = MTile{e, i * bm};
    }
    roff += rows[q];
    toff += tiles[q];
  }
  if (b == 0 && tid == kTokBlock - 1) {
    offsets[E] = roff;
    meta[kMetaMTiles] = toff;
    meta[kMetaRows] = roff;
  }
  if constexpr (!kOneBlock) mark();
  __syncthreads();              // s_off (and the masks) complete before any thread reads them
  if (!valid) return;
  for (int j = 0; j < k; ++j) {
    const int e = ids[t * k + j];
    if (!slot_kept(ids + t * k, j, e, E, kept)) continue;
    const uint32_t* m = mask + e * (kTokBlock / 32);
    int rank = __popc(m[word] & (bit - 1u));
    for (int w = 0; w < word; ++w) rank += __popc(m[w]);
    const int64_t r = static_cast<int64_t>(s_off[e]) + s_pre[e] + rank;
    row_tok[r] = static_cast<int32_t>(t);
    row_slot[r] = static_cast<int32_t>(t * k + j);
  }
}

struct PtrPairs {                 // kernel-argument batch of table entries
  int32_t n;
  int32_t idx[128];
  const void* ptr[128];
};

__global__ void upload_ptrs_kernel(const void** table, PtrPairs b) {
  const int i = threadIdx.x;
  if (i < b.n) table[b.idx[i]] = b.ptr[i];
}

}  // namespace

hipError_t launch_upload_ptrs(const void** table, const void* const* src, int first, int n,
                              hipStream_t s) {
  ProfScope prof(MOE_STAGE_TABLE, s);
  for (int i0 = 0; i0 < n; i0 += 128) {
    PtrPairs b{};
    b.n = std::min(128, n - i0);
    for (int i = 0; i < b.n; ++i) {
      b.idx[i] = first + i0 + i;
      b.ptr[i] = src[i0 + i];
    }
    upload_ptrs_kernel<<<1, 128, 0, s>>>(table, b);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

hipError_t launch_upload_pairs(const void** table, const int32_t* idx, const void* const* ptr,
                               int n, hipStream_t s) {
  ProfScope prof(MOE_STAGE_TABLE, s);
  for (int i0 = 0; i0 < n; i0 += 128) {
    PtrPairs b{};
    b.n = std::min(128, n - i0);
    for (int i = 0; i < b.n; ++i) {
      b.idx[i] = idx[i0 + i];
      b.ptr[i] = ptr[i0 + i];
    }
    upload_ptrs_kernel<<<1, 128, 0, s>>>(table, b);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

namespace {

// The bucketing launches for n_chunks chunks of seg.chunk tokens (grid.y = chunk): one
// permute-with-scan launch when a chunk is one token block; else the block histograms, then
// the scan inside the permute while a chunk has at most kScanBlocks blocks, or a scan launch
// and the permute.
hipError_t bucket_launches(const int32_t* ids, const ChunkSeg& seg, int n_chunks, int k, int E,
                           int bm, char* ws, const WsLayout& L, hipStream_t s) {
  const int nb = static_cast<int>((seg.chunk + kTokBlock - 1) / kTokBlock);
  int32_t* blk_counts = reinterpret_cast<int32_t*>(ws + L.blk_counts);
  int32_t* blk_base = reinterpret_cast<int32_t*>(ws + L.blk_base);
  int32_t* counts = reinterpret_cast<int32_t*>(ws + L.counts);
  int32_t* offsets = reinterpret_cast<int32_t*>(ws + L.offsets);
  int32_t* meta = reinterpret_cast<int32_t*>(ws + L.meta);
  MTile* mtiles = reinterpret_cast<MTile*>(ws + L.mtiles);
  int32_t* row_tok = reinterpret_cast<int32_t*>(ws + L.row_tok);
  int32_t* row_slot = reinterpret_cast<int32_t*>(ws + L.row_slot);
  const dim3 grid(static_cast<unsigned>(nb), static_cast<unsigned>(n_chunks));
  hipError_t err;
  if (nb == 1) {                // one launch: the block counts from its own masks
    ProfScope prof(MOE_STAGE_PERMUTE, s);
    permute_scan_kernel<true><<<grid, kTokBlock, 0, s>>>(ids, k, E, bm, blk_counts, counts,
                                                         offsets, mtiles, meta, row_tok,
                                                         row_slot, seg);
    return hipGetLastError();
  }
  {
    ProfScope prof(MOE_STAGE_HIST, s);
    block_hist_kernel<<<grid, kTokBlock, 0, s>>>(ids, k, E, blk_counts, seg);
    err = hipGetLastError();
  }
  if (err != hipSuccess) return err;
  if (nb <= kScanBlocks) {
    ProfScope prof(MOE_STAGE_PERMUTE, s);
    permute_scan_kernel<false><<<grid, kTokBlock, 0, s>>>(ids, k, E, bm, blk_counts, counts,
                                                          offsets, mtiles, meta, row_tok,
                                                          row_slot, seg);
    return hipGetLastError();
  }
  {
    ProfScope prof(MOE_STAGE_SCAN, s);
    scan_kernel<<<dim3(1, static_cast<unsigned>(n_chunks)), 1024, 0, s>>>(
        blk_counts, E, bm, blk_base, counts, offsets, mtiles, meta, seg);
    err = hipGetLastError();
  }
  if (err != hipSuccess) return err;
  ProfScope prof(MOE_STAGE_PERMUTE, s);
  permute_kernel<<<grid, kTokBlock, 0, s>>>(ids, k, E, blk_base, offsets, row_tok, row_slot,
                                            seg);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bucket(const int32_t* ids_chunk, int64_t n, int k, int E, int tile_rows,
                         char* ws, const WsLayout& L, hipStream_t s, int32_t* counts_out) {
  if (n <= 0) return hipSuccess;
  const ChunkSeg seg{n, n, 0, tile_rows, counts_out};
  return bucket_launches(ids_chunk, seg, 1, k, E, tile_rows, ws, L, s);
}

hipError_t launch_bucket_chunks(const int32_t* ids, int64_t T, int64_t chunk, int k, int E,
                                int tile_rows, int tile_rows_last, char* ws, const WsLayout& L,
                                int64_t stride, int32_t* counts_out, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const int64_t n_chunks = (T + chunk - 1) / chunk;
  const ChunkSeg seg{chunk, T, stride, tile_rows_last, counts_out};
  return bucket_launches(ids, seg, static_cast<int>(n_chunks), k, E, tile_rows, ws, L, s);
}

}  // namespace moe
