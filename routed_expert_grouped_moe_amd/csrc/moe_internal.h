// Internal declarations shared by the HIP translation units of libmoeprefill.
// Not part of the ABI: the exported surface is include/moe_prefill.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe_prefill.h"

#define MOE_HIDDEN __attribute__((visibility("hidden")))

namespace moe {

// ------------------------------------------------------------------ tiling constants
constexpr int kMinTileRows = 16;  // smallest M-tile height of the routed GEMMs
constexpr int kTokBlock = 256;    // tokens per block of the bucketing kernels
constexpr int kDecodeTileRows = 16;   // routed M-tile height below 16 rows per expert
// Chunks of at most this many tokens on decode tiles run the shared expert's tiles (16-row
// blocks) inside the routed launches and the stand-alone combine after them.
constexpr int kMixedDecodeRows = 192;
// In a layer call, chunks on decode tiles of up to this many tokens (and more than
// kMixedDecodeRows) defer their shared down + combine to the next chunk's gate/up launch, which
// also runs their shared gate/up as 16-row blocks.
constexpr int kDeferDecodeRows = 512;

// ------------------------------------------------------------------ device-side records
struct MTile {                    // one M-tile of a routed expert: rows [m0, m0 + tile rows)
  int32_t group;
  int32_t m0;
};

// Workspace layout for chunks of up to max_n tokens (all offsets 256-byte aligned).
struct WsLayout {
  size_t wtab, blk_counts, blk_base, counts, offsets, meta, mtiles, row_tok, row_slot;
  size_t h, h_shared, y, s_small, total;
  int64_t max_n, max_rows, max_mtiles, n_blocks;
};
MOE_HIDDEN bool ws_layout(const moe_shape& sh, int64_t max_n, WsLayout* out);

// moe_prefill_chunk after its argument checks. resident_only: a layer with offloaded experts is
// MOE_ERR_UNSUPPORTED. ws_of_device: when given, the workspace is ws_bytes of library-owned
// device memory whose address this returns for the current device (NULL with *status set on
// failure); it is asked for only after every argument check has passed.
MOE_HIDDEN moe_status prefill_chunk_checked(const moe_layer* layer, const void* x,
                                            const int32_t* ids, const float* weights, int64_t T,
                                            int64_t t0, int64_t n, const int32_t* counts_host,
                                            void* out, void* ws, size_t ws_bytes, void* stream,
                                            void* copy_stream, bool resident_only,
                                            void* (*ws_of_device)(moe_status*));

// meta words in the workspace
enum { kMetaMTiles = 0, kMetaRows = 1, kMetaWords = 64 };

// ------------------------------------------------------------------ launch wrappers
// (each returns hipGetLastError() after its launches)
MOE_HIDDEN hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s);

MOE_HIDDEN hipError_t launch_router_gemm(int dtype, const void* x, const void* w_router,
                                         const float* bias, int64_t T, int d, int E,
                                         float* logits, hipStream_t s);
// Also zeroes n_zero ints at `zero` (the per-chunk counts launch_chunk_hist then adds to).
MOE_HIDDEN hipError_t launch_topk(const float* logits, int64_t T, int E, int k, int32_t* ids,
                                  float* weights, int32_t* zero, int64_t n_zero, hipStream_t s);
// Top-k and the per-chunk counts of a prompt of at most 16 tokens in one launch
// (topk_counts_fused(T)); zeroes the n_cc counts itself.
MOE_HIDDEN bool topk_counts_fused(int64_t T);
MOE_HIDDEN hipError_t launch_topk_counts_small(const float* logits, int64_t T, int E, int k,
                                               int32_t* ids, float* weights, int64_t chunk,
                                               int32_t* chunk_counts, int64_t n_cc,
                                               hipStream_t s);
// chunk_counts must be zero on entry (launch_topk zeroes them).
MOE_HIDDEN hipError_t launch_chunk_hist(const int32_t* ids, int64_t T, int k, int E,
                                        int64_t chunk, int32_t* chunk_counts, hipStream_t s);

// Copy `bytes` (a multiple of 16; both pointers 16-byte aligned) from the device mapping of
// pinned host memory into device memory with a kernel on stream s.
MOE_HIDDEN hipError_t launch_line_copy(void* dst, const void* src_dev, size_t bytes,
                                       hipStream_t s);

MOE_HIDDEN hipError_t launch_upload_ptrs(const void** dst_table, const void* const* src,
                                         int first, int n, hipStream_t s);
MOE_HIDDEN hipError_t launch_upload_pairs(const void** table, const int32_t* idx,
                                         const void* const* ptr, int n, hipStream_t s);
// Bucketing of a chunk's slots by expert into the workspace (counts, offsets, M-tiles, member
// lists); counts_out (if not NULL) receives the chunk's expert counts as well.
MOE_HIDDEN hipError_t launch_bucket(const int32_t* ids_chunk, int64_t n, int k, int E,
                                    int tile_rows, char* ws, const WsLayout& L, hipStream_t s,
                                    int32_t* counts_out = nullptr);
// The same for every chunk of a prompt of T tokens in one set of launches: chunk c's lists go
// to the list offsets of L (a layout for chunks of `chunk` tokens) plus c * stride bytes, its
// M-tiles are tile_rows tall (tile_rows_last for the last chunk), and counts_out [chunks, E]
// (if not NULL) receives every chunk's expert counts.
MOE_HIDDEN hipError_t launch_bucket_chunks(const int32_t* ids, int64_t T, int64_t chunk, int k,
                                           int E, int tile_rows, int tile_rows_last, char* ws,
                                           const WsLayout& L, int64_t stride,
                                           int32_t* counts_out, hipStream_t s);

// M-tile height of the routed GEMMs for a chunk of n tokens: 320 when experts average 192 to
// 320 rows, 256 from 128 rows up otherwise, 128 from 48, 64 from 16 and 16 (decode tiles)
// below. The choice changes speed only, never a result bit.
MOE_HIDDEN int routed_tile_rows(int64_t n, int k, int E);

struct GemmGroups {               // routed (grouped) problem description
  const MTile* mtiles;
  const int32_t* n_mtiles;        // device scalar
  const int32_t* offsets;         // [E+1]
  const int32_t* counts;          // [E]
  const void* const* wtab;        // [E] expert line pointers (used when lines0 is NULL)
  const char* lines0;             // else line e starts at lines0 + e * line_stride
  int64_t line_stride;            // bytes
  int tile_lo;                    // first M-tile of this launch
  int tile_cap;                   // M-tiles this launch may cover (upper bound)
  int tile_rows;                  // M-tile height the tile list was built with
};

MOE_HIDDEN hipError_t launch_gu_routed(int dtype, const void* x, int64_t t0, int d, int I,
                                       const GemmGroups& g, const int32_t* row_tok, void* h,
                                       hipStream_t s);
MOE_HIDDEN hipError_t launch_gu_dense(int dtype, const void* x, int64_t t0, int64_t n, int d,
                                      int Is, const void* w_gu, void* h, hipStream_t s);
// The shared expert's gate/up GEMM and the routed one in one launch (routed M-tiles of
// tile_rows rows for a chunk of n tokens, for which gu_mixed_supported holds: 320-, 256-, 128-
// or 64-row tiles, or decode tiles for a chunk of at most kMixedDecodeRows tokens, whose shared
// rows then run as 16-row blocks).
MOE_HIDDEN bool gu_mixed_supported(int tile_rows, int64_t n);
MOE_HIDDEN hipError_t launch_gu_mixed(int dtype, const void* x, int64_t t0, int64_t n, int d,
                                      int I, int Is, const void* w_gu_shared, void* h_shared,
                                      const GemmGroups& g, const int32_t* row_tok, void* h,
                                      hipStream_t s);
// launch_gu_mixed with the previous chunk's shared down GEMM and combine (prev_n rows from
// prev_t0, its h_shared rows in prev_h_shared, its Y in y; prev_n == 0: none) in the same
// launch. For 256-, 128- and 64-row routed tiles (gu_mixed_combine_supported; 64-row ones for
// more than 16 tokens) and decode tiles for kMixedDecodeRows + 1 to kDeferDecodeRows tokens.
// h_shared must not be prev_h_shared: this chunk's gate/up writes it while the previous
// chunk's down GEMM reads that one.
MOE_HIDDEN bool gu_mixed_combine_supported(int tile_rows, int64_t n);
MOE_HIDDEN hipError_t launch_gu_mixed_combine(int dtype, const void* x, int64_t t0, int64_t n,
                                              int d, int I, int Is, const void* w_gu_shared,
                                              void* h_shared, const GemmGroups& g,
                                              const int32_t* row_tok, void* h,
                                              const void* prev_h_shared, int64_t prev_t0,
                                              int64_t prev_n, const void* w_down_shared,
                                              const float* y, const float* weights, int k,
                                              void* out, hipStream_t s);
MOE_HIDDEN hipError_t launch_down_routed(int dtype, const void* h, int d, int I,
                                         const GemmGroups& g, const int32_t* row_slot,
                                         float* y, hipStream_t s);
// Both routed GEMMs of each M-tile in one workgroup, h kept in LDS (bf16, 64-row tiles, I a
// multiple of 128 up to 512: gu_down_fused_supported); writes Y only, not h.
MOE_HIDDEN bool gu_down_fused_supported(int dtype, int tile_rows, int I);
MOE_HIDDEN hipError_t launch_gu_down_fused(const void* x, int64_t t0, int d, int I,
                                           const GemmGroups& g, const int32_t* row_tok,
                                           const int32_t* row_slot, float* y, hipStream_t s);
// The shared expert's down GEMM with the combine folded in: out rows t0 .. t0 + n - 1.
MOE_HIDDEN hipError_t launch_down_combine(int dtype, const void* h, int64_t n, int d, int Is,
                                          const void* w_down, const float* y,
                                          const float* weights, int64_t t0, int k, void* out,
                                          hipStream_t s);
// The shared expert's down GEMM (S alone) and the routed one in one launch, for a chunk of at
// most kMixedDecodeRows tokens on decode tiles (g.tile_rows == 16).
MOE_HIDDEN hipError_t launch_down_mixed(int dtype, const void* h_shared, int64_t n, int d,
                                        int Is, const void* w_down_shared, float* s_out,
                                        const void* h, int I, const GemmGroups& g,
                                        const int32_t* row_slot, float* y, hipStream_t s);
MOE_HIDDEN hipError_t launch_combine(int dtype, const float* y, const float* shared,
                                     const float* weights, int64_t t0, int64_t n, int k, int d,
                                     void* out, hipStream_t s);
MOE_HIDDEN hipError_t launch_add_rmsnorm(int dtype, const void* x, const void* delta,
                                         int64_t T, int d, float eps, void* x_out,
                                         void* normed, hipStream_t s);

// number of M-tiles of a group with c rows
inline int64_t mtiles_of(int64_t c, int tile_rows) { return (c + tile_rows - 1) / tile_rows; }

}  // namespace moe
