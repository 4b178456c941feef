// GEMMs of the layer on CDNA4 matrix cores: the router, each expert's gate/up projection with
// the fused silu(gate)*up epilogue, each expert's down projection, and the shared expert's
// down projection with the combine in its epilogue.
//
// Every GEMM here is X W^T with both operands K-contiguous (token rows and weight rows). A
// workgroup computes a BM x BN tile; K advances 128 bytes per row and stage (64 bf16 or 32
// fp32 elements) through two LDS stages (three in the router's tile, four in the decode tile)
// filled by direct global->LDS loads (global_load_lds_dwordx4: each lane's 16 bytes land at
// the instruction's LDS base plus 16 x lane, so one instruction fills 8 rows of 128 bytes; the
// stage's instructions go round-robin over the waves, so every wave loads a share of both
// operands; the A rows of a routed tile are gathered from the prompt by pointer, no permuted
// copy of x exists). The A stage buffers sit together in LDS, followed by the B ones. Inside LDS, 16-byte segment g of row r sits at segment g ^ (r & 7), so any 8
// consecutive lanes reading one MFMA operand (8 rows, same K segment) hit 8 different bank
// groups. A wave row-group owns every WM-th 16-row block of the tile and accumulates
// 16 x 16 MFMA blocks: v_mfma_f32_16x16x32_bf16 (bf16) or v_mfma_f32_16x16x4_f32 (fp32),
// fp32 accumulation.
//
// Tile shapes: tall (320 x 256, 8 waves of 80 x 128) and big (256 x 256, 8 waves of 64 x 128)
// for large row counts; mid (128 x 256, 8 waves of 64 x 64, three stage buffers) for experts
// of 48 to 128 rows and mid-sized dense GEMMs; small (64 x 256, 4 waves of 64 x 64; two or,
// for short dense GEMMs, four stage buffers) for fewer rows, and its narrow variant (64 x
// 128) for the shortest dense GEMMs; decode (16 x 64, one wave) for calls of a few tokens. Which one runs never changes a bit: every output element is one
// token row against one weight row, accumulated over K in the same stage order with the same
// instruction and the same lane-to-K mapping in all of them. Together with no split-K, no
// atomics and no shape-dependent arithmetic, that is what makes a token's bytes independent
// of the chunk size, of its position and of its expert's row count -- the property the exact
// deep prefill page ("Flash Next EXL3: exact deep prefill", opening section) asks of its
// GU/down kernels.
#include <type_traits>

#include "device_common.h"
#include "moe_internal.h"
#include "profile.h"

namespace moe {
namespace {

// RB_: K bytes per row and stage, 128 (64 bf16 / 32 fp32 elements) or 64. A 1 KB load
// instruction fills RPL = 1024 / RB rows, and the stage's NBLK instructions go round-robin
// over the waves (block b to wave b % NW): the A blocks come first and every wave issues QA of
// them, then the B blocks (with NBLK not a multiple of NW the first FULL waves issue one more).
// LDS holds the NBUF stage buffers of the A rows, then the NBUF stage buffers of the B rows.
template <int BM_, int BN_, int WM_, int WN_, int NBUF_ = 2, int RB_ = 128>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr int NBUF = NBUF_;                        // LDS stage buffers (NBUF - 1 in flight)
  static constexpr int RB = RB_;
  static constexpr int NW = WM * WN, NT = 64 * NW;
  static constexpr int TM = BM / WM, TN = BN / WN;          // wave tile
  static constexpr int FM = TM / 16, FN = TN / 16;          // 16 x 16 MFMA blocks per wave
  static constexpr int ROWS = BM + BN;
  static constexpr int A_STAGE = BM * RB, B_STAGE = BN * RB;
  static constexpr int B_OFF = NBUF * A_STAGE;              // first B stage buffer
  static constexpr int LDS = NBUF * (A_STAGE + B_STAGE);
  static constexpr int SPR = RB / 16;                       // 16-byte segments per row
  static constexpr int RPL = 1024 / RB;                     // rows per load instruction
  static constexpr int NBLK = ROWS / RPL;                   // load instructions per stage
  static constexpr int QA = BM / RPL / NW;                  // A load instructions per wave
  static constexpr int LPW = (NBLK + NW - 1) / NW;          // per wave, at most
  static constexpr int FULL = NBLK - (LPW - 1) * NW;        // waves that issue LPW
  static_assert(NBUF >= 2 && NBUF <= 4, "two to four stage buffers");
  static_assert(RB == 128 || RB == 64, "64 or 128 K bytes per row and stage");
  static_assert(TM % 16 == 0 && TN % 16 == 0, "whole 16 x 16 MFMA blocks per wave");
  static_assert(ROWS % RPL == 0, "whole load instructions per stage");
  static_assert((BM / RPL) % NW == 0 && QA < LPW, "every wave loads whole A blocks and some B");
  static_assert(LDS <= 160 * 1024, "LDS of one CU");
};
using BigTile = Tile<256, 256, 4, 2>;      // 8 waves, 64 x 128 each; 128 KB LDS, 1 workgroup/CU
using TallTile = Tile<320, 256, 4, 2>;     // 8 waves, 80 x 128 each; 144 KB LDS, 1 workgroup/CU
using SmallTile = Tile<64, 256, 1, 4>;     // 4 waves, 64 x 64 each; 80 KB LDS, 2 workgroups/CU
// Dense GEMMs with at most one small tile per CU: four stage buffers (three stages in
// flight), 160 KB LDS, 1 workgroup/CU
using SmallTile4 = Tile<64, 256, 1, 4, 4>;
// ... and at most half a tile per CU: half as wide (4 waves of 64 x 32), twice the tiles, 96 KB
using NarrowTile4 = Tile<64, 128, 1, 4, 4>;
using MidTile = Tile<128, 256, 2, 4, 3>;   // 8 waves, 64 x 64 each; 3 stage buffers, 144 KB LDS, 1 workgroup/CU
// Decode-sized calls: a GEMM of at most 16 rows has few tiles, and each walks its K stages one
// round trip at a time; narrow one-wave tiles with three stages in flight (40 KB LDS).
using DecodeTile = Tile<16, 64, 1, 1, 4>;
// Routers of short prompts: with few rows, tiles narrow in N give the chip more workgroups,
// each with its own stage loads in flight. 16x16 one-wave tiles (16 KB LDS) while they make at
// most 128 workgroups (and always for at most 16 rows), then 64x64 tiles of four waves of
// 64x16 (64 KB) while they make at most 512.
using RouterTile16 = Tile<16, 16, 1, 1, 4>;
using RouterTile64 = Tile<64, 64, 1, 4, 4>;
// The shared expert's GEMMs of short prompts (17 to 512 rows) for the same reason: decode tiles
// over 16-row blocks up to 64 rows, then 64x64 tiles (the down GEMM on RouterTile64; the
// gate/up on two waves of 64x32, so that each wave holds the gate and the up half of its h
// columns).
using PairTile64 = Tile<64, 64, 1, 2, 4>;

// Segment swizzle of tile row r (16-row blocks start at multiples of 16, so a lane's row
// within its MFMA block decides it): 16-byte segment g of the row sits at g ^ swz(r). For
// 128-byte rows that is r & 7, for 64-byte rows (r >> 2) & 3; either way any 8 consecutive
// lanes reading one MFMA operand (8 rows, one segment) hit 8 different bank groups.
template <class TL>
__device__ __forceinline__ int swz(int r) {
  return TL::RB == 128 ? (r & 7) : ((r >> 2) & 3);
}

// Wave rows: wave row-group wm owns the tile's 16-row blocks wm, wm + WM, wm + 2 WM, ...
// (block i of the wave starts at tile row (i * WM + wm) * 16). Interleaving keeps the work of
// a partly filled tile spread over all SIMDs; blocks past the tile's valid rows are skipped.
template <class TL>
__device__ __forceinline__ int block_row(int i, int wm) {
  return (i * TL::WM + wm) * 16;
}
// Number of this wave's blocks that hold valid rows (they are a prefix of its blocks).
template <class TL>
__device__ __forceinline__ int busy_blocks(int rows, int wm) {
  const int r16 = (rows + 15) / 16;
  return r16 > wm ? min(TL::FM, (r16 - wm + TL::WM - 1) / TL::WM) : 0;
}

// s_waitcnt vmcnt(N) leaving the other counters alone (gfx9 encoding of the immediate).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <typename T> struct Frag;

// bf16: a 64-byte MFMA step holds 32 K elements. Lane l supplies row (l & 15) and the 8
// consecutive K elements of 16-byte segment (4 * step + (l >> 4)), for A and B alike.
template <> struct Frag<uint16_t> {
  static constexpr int kStepBytes = 64;
  typedef bf16x8_t V;
  static __device__ __forceinline__ V load(const char* row, int step, int kq, int sw) {
    return *reinterpret_cast<const V*>(row + (((step * 4 + kq) ^ sw) << 4));
  }
  static __device__ __forceinline__ f32x4_t mma(V a, V b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

// fp32: a 16-byte MFMA step holds 4 K elements; lane l supplies element (l >> 4) of the
// step, i.e. 4-byte word (l >> 4) of 16-byte segment `step`.
template <> struct Frag<float> {
  static constexpr int kStepBytes = 16;
  typedef float V;
  static __device__ __forceinline__ V load(const char* row, int step, int kq, int sw) {
    return *reinterpret_cast<const V*>(row + (((step ^ sw) << 4) | (kq << 2)));
  }
  static __device__ __forceinline__ f32x4_t mma(V a, V b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

// Row this lane stages for load instruction q (block wave + NW q of the stage), and the
// segment of it that it loads, so that after the swizzle the instruction's 1 KB holds RPL
// whole rows. Rows past ROWS (q beyond this wave's share) are never loaded.
template <class TL>
__device__ __forceinline__ int stage_row(int q) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  return (wave + TL::NW * q) * TL::RPL + lane / TL::SPR;
}
template <class TL>
__device__ __forceinline__ int stage_seg() {
  const int lane = threadIdx.x & 63;
  return (lane % TL::SPR) ^ swz<TL>(lane / TL::SPR);
}

// K stages of a GEMM with K elements of type T.
template <typename T, class TL>
__host__ __device__ constexpr int stages(int K) {
  return K / (TL::RB / static_cast<int>(sizeof(T)));
}

// Mainloop. src[q]: this lane's global source (row start + 16 * stage_seg<TL>()) for load
// instruction q; stage s reads TL::RB bytes further per stage. kPairedGU: the B half holds
// BN/2 gate rows then the BN/2 matching up rows; wave column wn takes gate blocks wn*TN/2..
// and the up blocks of the same columns, so acc[i][j] and acc[i][j + FN/2] are gate and up of
// one output element. rows: valid rows of the tile; a wave keeps loading its share of the
// stages but skips the fragment reads and MFMAs of its blocks past `rows` (their outputs are
// never stored). kSpread: the next stage's loads go out between the MFMA rows of the first K
// step instead of all at once after the barrier.
template <typename T, class TL, bool kPairedGU, bool kSpread = false>
__device__ __forceinline__ void mainloop(const char* const (&src)[TL::LPW], int nk, char* lds,
                                         f32x4_t (&acc)[TL::FM][TL::FN], int rows) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / TL::WN, wn = wave % TL::WN, kq = lane >> 4, l16 = lane & 15;
  const int nbusy = busy_blocks<TL>(rows, wm);
  const int sw = swz<TL>(l16);
  constexpr int kSteps = TL::RB / Frag<T>::kStepBytes;     // MFMA K steps per stage
  int arow[TL::FM], brow[TL::FN];
#pragma unroll
  for (int i = 0; i < TL::FM; ++i) arow[i] = (block_row<TL>(i, wm) + l16) * TL::RB;
#pragma unroll
  for (int j = 0; j < TL::FN; ++j) {
    int b;
    if (kPairedGU) {
      constexpr int H = TL::FN / 2;
      b = (j < H) ? wn * (TL::TN / 2) + j * 16 : TL::BN / 2 + wn * (TL::TN / 2) + (j - H) * 16;
    } else {
      b = wn * TL::TN + j * 16;
    }
    brow[j] = (b + l16) * TL::RB;
  }
#pragma unroll
  for (int i = 0; i < TL::FM; ++i)
#pragma unroll
    for (int j = 0; j < TL::FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // The stage loads are issued as inline asm (M0 = the instruction's 1 KB LDS block, one
  // global_load_lds_dwordx4 each) so the compiler does not track them: the only waits they
  // need are the explicit vmcnt waits before each stage's barrier, and with them out of its
  // bookkeeping the compiler waits on each fragment read separately (lgkmcnt(N)) instead of
  // on all of them (lgkmcnt(0)) -- 5-9% faster mainloops, same instructions.
  typedef __attribute__((address_space(3))) char lds_char;
  const int uwave = __builtin_amdgcn_readfirstlane(wave);
  const bool full = TL::FULL == TL::NW || uwave < TL::FULL;   // issues LPW loads, else LPW - 1
  const uint32_t wave_lds = __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>((uintptr_t)(lds_char*)lds) + static_cast<uint32_t>(uwave * 1024));
  // Spread issue: after MFMA row i < FM - 1 of the first K step comes slot i with its share of
  // the next stage's LPW load instructions, so a wave does not sit on a full load queue with its
  // MFMAs waiting behind. That pays where the operands are mostly cache hits (the dense shared
  // GU: 236 against 261 us at T = 16,022); the routed GEMMs, whose gathered rows and weights
  // come from HBM, need every cycle of lead time and issue at once after the barrier.
  constexpr int kSlots = TL::FM - 1;
  constexpr bool kSpreadOn = kSpread && kSlots > 0;
  // M0 is a reserved register to the compiler (hence the silenced warning); no other code in
  // these kernels uses it, which tests/test_isa_guard.py checks on the compiled ISA.
  auto issue_q = [&](uint32_t dst, int q, int s) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(dst)),
                   "v"(src[q] + k_stage<TL::BM>(s, nk) * TL::RB)
                 : "memory", "m0");
#pragma clang diagnostic pop
  };
  auto issue_part = [&](int s, int qlo, int qhi) {
    const uint32_t da = wave_lds + static_cast<uint32_t>((s % TL::NBUF) * TL::A_STAGE);
    const uint32_t db = wave_lds + static_cast<uint32_t>(TL::B_OFF + (s % TL::NBUF) * TL::B_STAGE);
#pragma unroll
    for (int q = 0; q < TL::LPW; ++q) {
      if (q >= qlo && q < qhi && (q < TL::LPW - 1 || full)) {
        if (q < TL::QA) issue_q(da + static_cast<uint32_t>(q * TL::NW * 1024), q, s);
        else issue_q(db + static_cast<uint32_t>((q - TL::QA) * TL::NW * 1024), q, s);
      }
    }
  };
  // issue(s, qlo, qhi): this wave's load instructions qlo .. qhi - 1 of stage s (issued from
  // inside the MFMA rows with a scheduling fence on either side, so they stay where they are)
  auto issue = [&](int s, int qlo, int qhi) {
    if constexpr (kSpreadOn) __builtin_amdgcn_sched_barrier(0);
    issue_part(s, qlo, qhi);
    if constexpr (kSpreadOn) __builtin_amdgcn_sched_barrier(0);
  };
  auto issue_slot = [&](int s, int m) {
    if constexpr (kSpreadOn)
      issue(s, (m * TL::LPW + kSlots - 1) / kSlots, ((m + 1) * TL::LPW + kSlots - 1) / kSlots);
  };
  // Two copies of the stage loop: every block valid (straight-line fragment reads, then the
  // MFMAs), or a partly valid wave that skips the blocks past `rows` (uniform branches).
  // With NBUF buffers, stages s + 1 .. s + NBUF - 2 stay in flight while stage s is waited
  // for (a wave's loads complete in issue order, so vmcnt(ahead x its loads per stage) is
  // enough).
  auto wait_ahead = [&](auto per_stage, int ahead) {
    constexpr int L = decltype(per_stage)::value;
    if (ahead >= 2) wait_vmcnt<2 * L>();
    else if (ahead == 1) wait_vmcnt<L>();
    else wait_vmcnt<0>();
  };
  auto wait_stage = [&](int s) {
    if constexpr (TL::NBUF == 2) {
      wait_vmcnt<0>();
    } else {
      const int ahead = min(TL::NBUF - 2, nk - 1 - s);
      if (full) wait_ahead(std::integral_constant<int, TL::LPW>{}, ahead);
      else wait_ahead(std::integral_constant<int, TL::LPW - 1>{}, ahead);
    }
  };
  auto run = [&](auto guarded) {
    for (int s = 0; s < TL::NBUF - 1 && s < nk; ++s) issue(s, 0, TL::LPW);
    for (int s = 0; s < nk; ++s) {
      wait_stage(s);              // this wave's share of stage s has landed ...
      __syncthreads();            // ... and everyone's; everyone also left stage s - 1
      const int sn = s + TL::NBUF - 1;           // stage whose loads go out now
      const bool pre = sn < nk;
      if (!kSpreadOn && pre) issue(sn, 0, TL::LPW);
      const char* abuf = lds + (s % TL::NBUF) * TL::A_STAGE;
      const char* bbuf = lds + TL::B_OFF + (s % TL::NBUF) * TL::B_STAGE;
      if constexpr (!decltype(guarded)::value) {
#pragma unroll
        for (int ks = 0; ks < kSteps; ++ks) {
          typename Frag<T>::V a[TL::FM], b[TL::FN];
#pragma unroll
          for (int i = 0; i < TL::FM; ++i) a[i] = Frag<T>::load(abuf + arow[i], ks, kq, sw);
#pragma unroll
          for (int j = 0; j < TL::FN; ++j) b[j] = Frag<T>::load(bbuf + brow[j], ks, kq, sw);
#pragma unroll
          for (int i = 0; i < TL::FM; ++i) {
#pragma unroll
            for (int j = 0; j < TL::FN; ++j) acc[i][j] = Frag<T>::mma(a[i], b[j], acc[i][j]);
            if (ks == 0 && i < TL::FM - 1 && pre) issue_slot(sn, i);
          }
        }
      } else if (nbusy > 0) {
#pragma unroll
        for (int ks = 0; ks < kSteps; ++ks) {
          typename Frag<T>::V b[TL::FN];
#pragma unroll
          for (int j = 0; j < TL::FN; ++j) b[j] = Frag<T>::load(bbuf + brow[j], ks, kq, sw);
#pragma unroll
          for (int i = 0; i < TL::FM; ++i) {
            if (i < nbusy) {
              const typename Frag<T>::V a = Frag<T>::load(abuf + arow[i], ks, kq, sw);
#pragma unroll
              for (int j = 0; j < TL::FN; ++j) acc[i][j] = Frag<T>::mma(a, b[j], acc[i][j]);
            }
            if (ks == 0 && i < TL::FM - 1 && pre) issue_slot(sn, i);
          }
        }
      } else if (pre && kSpreadOn) {
        issue(sn, 0, TL::LPW);                  // no rows of this wave: all loads at once
      }
    }
  };
  if (nbusy == TL::FM)
    run(std::false_type{});
  else
    run(std::true_type{});
  __syncthreads();              // LDS free for the epilogue
}

// Accumulator element acc[i][j][r] of a lane sits at row 4*(lane >> 4) + r of the wave's block
// i (tile row block_row(i, wm) + 4*(lane >> 4) + r) and at wave column j*16 + (lane & 15).

// XCD-aware placement of a 1-D grid. Workgroups are handed to the 8 XCDs round-robin
// (workgroup w runs on XCD w % 8), and each XCD has its own L2. Workgroup w takes tile
// (w % 8) * q + w / 8 with q = ceil(n_tiles / 8): every XCD works through one contiguous
// slice of the tile sequence, so the tiles that share weights or activation rows (neighbours
// in the sequence) meet in the same L2. The grid is padded to a multiple of 8; surplus
// workgroups have no tile.
constexpr int kXcds = 8;
__device__ __forceinline__ bool xcd_tile(int n_tiles, int* t) {
  const int w = static_cast<int>(blockIdx.x);
  const int q = (n_tiles + kXcds - 1) / kXcds;
  const int j = w / kXcds;
  const int tt = (w % kXcds) * q + j;
  if (j >= q || tt >= n_tiles) return false;
  *t = tt;
  return true;
}
inline unsigned xcd_grid(int64_t n_tiles) {
  return static_cast<unsigned>((n_tiles + kXcds - 1) / kXcds * kXcds);
}
// Two unit sequences in one launch: each XCD works through its contiguous slice of sequence A
// (na units), then its slice of sequence B (nb units), slices as in xcd_tile. Workgroups are
// dispatched in order, so A's units start first on every XCD. The grid is
// xcd_grid(na) + xcd_grid(nb) (nb may be an upper bound: surplus workgroups have no unit).
__device__ __forceinline__ bool xcd_tile_two(int na, int nb, int* t, bool* in_a) {
  const int w = static_cast<int>(blockIdx.x);
  const int qa = (na + kXcds - 1) / kXcds, qb = (nb + kXcds - 1) / kXcds;
  const int x = w % kXcds, j = w / kXcds;
  const bool a = j < qa;
  const int tt = a ? x * qa + j : x * qb + (j - qa);
  if (tt >= (a ? na : nb) || (!a && j - qa >= qb)) return false;
  *t = tt;
  *in_a = a;
  return true;
}

// Output of one wave's blocks through LDS in 16-row rounds: the lanes write their accumulator
// values (transformed by `val`) into a per-wave staging area, then store whole rows with
// 16-byte vectors. row_of(16*i + r) maps row r of the wave's block i to its global output row
// (or -1 to skip),
// OUT is the stored element type, cols = columns of the slab that exist (<= NCOL).
template <class TL, typename OUT, int NCOL, bool kStreamOut = false, class Val, class RowOf>
__device__ __forceinline__ void store_slab(char* lds, Val val, RowOf row_of, OUT* out,
                                           int64_t ld, int col0, int cols) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int RB = NCOL * static_cast<int>(sizeof(OUT));        // bytes per staged row
  constexpr int CPR = RB / 16;                                      // 16-byte chunks per row
  OUT* stg = reinterpret_cast<OUT*>(lds + wave * (16 * RB));
  static_assert(16 * RB * TL::NW <= TL::LDS, "staging fits in LDS");
#pragma unroll
  for (int i = 0; i < TL::FM; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int j = 0; j < NCOL / 16; ++j)
        stg[(4 * (lane >> 4) + r) * NCOL + j * 16 + (lane & 15)] = val(i, j, r);
    __builtin_amdgcn_wave_barrier();
    constexpr int EPC = 16 / static_cast<int>(sizeof(OUT));       // elements per chunk
    // 16-byte stores need 16-byte aligned rows; a chunk that would cross `cols` (or a row
    // pitch that is not a multiple of 16 bytes) goes element by element
    const bool vec = (ld % EPC) == 0 && (col0 % EPC) == 0 &&
                     (reinterpret_cast<uintptr_t>(out) & 15) == 0;
#pragma unroll
    for (int c = lane; c < 16 * CPR; c += 64) {
      const int row = c / CPR, ch = c % CPR;
      const int64_t grow = row_of(i * 16 + row);
      const int col = ch * EPC;
      if (grow < 0 || col >= cols) continue;
      const char* s = reinterpret_cast<const char*>(stg) + row * RB + ch * 16;
      OUT* d = out + grow * ld + col0 + col;
      if (vec && col + EPC <= cols) {
        if (kStreamOut)   // written once, read once by another kernel: keep it out of the caches
          __builtin_nontemporal_store(*reinterpret_cast<const u32x4_t*>(s),
                                      reinterpret_cast<u32x4_t*>(d));
        else
          *reinterpret_cast<u32x4_t*>(d) = *reinterpret_cast<const u32x4_t*>(s);
      } else {
        for (int e = 0; e < EPC && col + e < cols; ++e) d[e] = reinterpret_cast<const OUT*>(s)[e];
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

struct GuParams {
  const void* x;          // [T, d] prompt rows
  int64_t t0;             // first prompt row of the chunk
  int64_t n;              // dense: rows of the chunk
  int d, I;               // K and h width
  const void* w;          // dense: [2I, d] gate/up weights
  GemmGroups g;           // grouped: routed experts
  const int32_t* row_tok; // grouped: chunk-local token of each permuted row
  void* h;                // [rows, I] out
  unsigned long long* clk;   // profiling clock counters of the stage, or NULL
};

// Clock sampling for the opt-in profiling: thread 0 of a workgroup notes the core clock and
// the 100 MHz real-time counter at its start and adds the differences at its end.
struct ClockSample {
  unsigned long long* clk;
  unsigned long long c0 = 0, r0 = 0;
  __device__ explicit ClockSample(unsigned long long* p) : clk(threadIdx.x == 0 ? p : nullptr) {
    if (clk) {
      c0 = __builtin_amdgcn_s_memtime();
      r0 = __builtin_amdgcn_s_memrealtime();
    }
  }
  __device__ void finish() {
    if (!clk) return;
    const unsigned long long c1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
    atomicAdd(clk, c1 - c0);
    atomicAdd(clk + 1, r1 - r0);
  }
};

// Start of expert e's line: from the uniform layout when there is one, else from the table.
__device__ __forceinline__ const char* line_of(const GemmGroups& g, int e) {
  return g.lines0 ? g.lines0 + static_cast<int64_t>(e) * g.line_stride
                  : static_cast<const char*>(g.wtab[e]);
}

// Work units (M-tile x N-tile) of a gate/up launch: grouped units come from the device's
// M-tile list, dense ones from the row count.
template <class TL, bool kGrouped>
__device__ __forceinline__ int gu_units(const GuParams& p) {
  constexpr int HC = TL::BN / 2;
  const int NT = (p.I + HC - 1) / HC;
  const int m_tiles = kGrouped ? max(0, min(p.g.tile_cap, *p.g.n_mtiles - p.g.tile_lo))
                               : static_cast<int>((p.n + TL::BM - 1) / TL::BM);
  return m_tiles * NT;
}

template <typename T, class TL, bool kGrouped>
__device__ __forceinline__ void gu_tile(const GuParams& p, int t, char* lds);

template <typename T, class TL, bool kGrouped>
__global__ __launch_bounds__(TL::NT) __attribute__((amdgpu_waves_per_eu(2)))
void gu_kernel(GuParams p) {
  __shared__ __attribute__((aligned(1024))) char lds[TL::LDS];
  int t;
  if (!xcd_tile(gu_units<TL, kGrouped>(p), &t)) return;
  gu_tile<T, TL, kGrouped>(p, t, lds);
}

// The shared expert's gate/up units and the routed ones in one launch (shared units first in
// the unit sequence). Each XCD works through its contiguous slice of that sequence, so while
// the slices of the routed units stream expert weights from HBM, others run the shared GEMM,
// whose operands come from the caches: the two overlap on the chip instead of running one
// after the other, and the shared units fill what would be the routed launch's partial last
// round. Same tile, instruction and K order as the separate launches: the same bits.
template <typename T, class TL>
__global__ __launch_bounds__(TL::NT) __attribute__((amdgpu_waves_per_eu(2)))
void gu_mixed_kernel(GuParams shared, GuParams routed) {
  __shared__ __attribute__((aligned(1024))) char lds[TL::LDS];
  const int ns = gu_units<TL, false>(shared);
  int t;
  if (!xcd_tile(ns + gu_units<TL, true>(routed), &t)) return;
  if (t < ns)
    gu_tile<T, TL, false>(shared, t, lds);
  else
    gu_tile<T, TL, true>(routed, t - ns, lds);
}

template <typename T, class TL, bool kGrouped>
__device__ __forceinline__ void gu_tile(const GuParams& p, int t, char* lds) {
  constexpr int HC = TL::BN / 2;                         // h columns per tile
  const int NT = (p.I + HC - 1) / HC;
  ClockSample clock(p.clk);
  const int mi = t / NT;
  const int n0h = (t % NT) * HC;
  int64_t row0;
  int rows;
  const char* wbase;
  if (kGrouped) {
    const MTile mt = p.g.mtiles[p.g.tile_lo + mi];
    row0 = static_cast<int64_t>(p.g.offsets[mt.group]) + mt.m0;
    rows = min(TL::BM, p.g.counts[mt.group] - mt.m0);
    wbase = line_of(p.g, mt.group);
  } else {
    row0 = static_cast<int64_t>(mi) * TL::BM;
    rows = static_cast<int>(min<int64_t>(TL::BM, p.n - row0));
    wbase = static_cast<const char*>(p.w);
  }
  const bool missing = wbase == nullptr;   // offloaded expert that was not staged
  const size_t rowb = static_cast<size_t>(p.d) * sizeof(T);
  const char* src[TL::LPW];
#pragma unroll
  for (int q = 0; q < TL::LPW; ++q) {
    const int r = stage_row<TL>(q);
    const char* base;
    if (r < TL::BM) {
      const int ar = r < rows ? r : 0;     // rows past the end compute and are dropped
      const int64_t tok = kGrouped ? p.row_tok[row0 + ar] : row0 + ar;
      base = static_cast<const char*>(p.x) + (p.t0 + tok) * rowb;
    } else {
      const int br = r - TL::BM;
      const int hc = n0h + (br < HC ? br : br - HC);
      const int wrow = (hc < p.I ? hc : n0h) + (br < HC ? 0 : p.I);
      base = (missing ? static_cast<const char*>(p.x) : wbase) + static_cast<int64_t>(wrow) * rowb;
    }
    src[q] = base + 16 * stage_seg<TL>();
  }
  f32x4_t acc[TL::FM][TL::FN];
  if (!missing)
    mainloop<T, TL, true, !kGrouped>(src, stages<T, TL>(p.d), lds, acc, rows);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / TL::WN, wn = wave % TL::WN;
  constexpr int H = TL::FN / 2;
  if (missing) {                // no weights for this expert: its h rows are NaN
    const float nan = __builtin_nanf("");
#pragma unroll
    for (int i = 0; i < TL::FM; ++i)
#pragma unroll
      for (int j = 0; j < TL::FN; ++j) acc[i][j] = f32x4_t{nan, nan, nan, nan};
  }
  auto val = [&](int i, int j, int r) -> T {
    return h_store<T>(silu_f32(acc[i][j][r]) * acc[i][j + H][r]);
  };
  auto row_of = [&](int sr) -> int64_t {      // sr = block * 16 + row in block
    const int tr = block_row<TL>(sr >> 4, wm) + (sr & 15);
    return tr < rows ? row0 + tr : -1;
  };
  const int col0 = n0h + wn * (TL::TN / 2);
  store_slab<TL, T, TL::TN / 2>(lds, val, row_of, static_cast<T*>(p.h), p.I, col0,
                                min(TL::TN / 2, p.I - col0));
  clock.finish();
}

// Epilogue of the shared expert's down GEMM with the combine folded in. The tile holds S
// (fp32) for its rows and columns; each (token, 4 columns) then gets
//   acc = 0; acc = fma(w_j, y_j, acc) for j = 0 .. k-1 (ascending expert); acc += S;
//   out = round(acc)
// with the operations and their order of combine_kernel, so the bits do not depend on which
// of the two formed them. A lane handles U 4-column chunks at a time, with the Y loads of all
// k slots of them in flight before their FMAs: two chunks, or one where the wave's accumulators
// already take 128 registers (the 64 x 128 wave tile), since two chunks' loads beside them
// would exceed 256 registers and spill (the reloads cost 7% of the 256 x 256 tile's time).
template <class TL, typename T, class Val>
__device__ __forceinline__ void combine_slab(char* lds, Val val, int wm, int64_t row0, int rows,
                                             const float* __restrict__ y,
                                             const float* __restrict__ wts, int64_t t0, int k,
                                             int d, T* __restrict__ out, int col0, int cols) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int NCOL = TL::TN, RB = NCOL * 4, CPR = RB / 16,
                U = (TL::FM * TL::FN * 4 >= 128 || 16 * CPR < 128) ? 1 : 2;
  static_assert(16 * RB * TL::NW <= TL::LDS, "staging fits in LDS");
  static_assert((16 * CPR) % (64 * U) == 0, "whole groups of U chunks per block");
  float* stg = reinterpret_cast<float*>(lds + wave * (16 * RB));
#pragma unroll
  for (int i = 0; i < TL::FM; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int j = 0; j < NCOL / 16; ++j)
        stg[(4 * (lane >> 4) + r) * NCOL + j * 16 + (lane & 15)] = val(i, j, r);
    __builtin_amdgcn_wave_barrier();
#pragma unroll 1
    for (int c0 = lane; c0 < 16 * CPR; c0 += 64 * U) {
      int64_t t[U];
      int col[U];
      bool on[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + 64 * u, row = c / CPR;
        const int tr = block_row<TL>(i, wm) + row;
        col[u] = (c % CPR) * 4;
        on[u] = tr < rows && col[u] < cols;
        t[u] = row0 + (on[u] ? tr : 0);
      }
      f32x4_t acc[U];
#pragma unroll
      for (int u = 0; u < U; ++u) acc[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      int j = 0;
      for (; j + 8 <= k; j += 8) {
        f32x4_t v[8][U];
#pragma unroll
        for (int q = 0; q < 8; ++q)
#pragma unroll
          for (int u = 0; u < U; ++u)
            v[q][u] = on[u] ? __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(
                                  y + (t[u] * k + MOE_SLOT(j + q, k)) * d + col0 + col[u]))
                            : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < 8; ++q)
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const float wj = wts[(t0 + t[u]) * k + MOE_SLOT(j + q, k)];
            acc[u][0] = fmaf(wj, v[q][u][0], acc[u][0]);
            acc[u][1] = fmaf(wj, v[q][u][1], acc[u][1]);
            acc[u][2] = fmaf(wj, v[q][u][2], acc[u][2]);
            acc[u][3] = fmaf(wj, v[q][u][3], acc[u][3]);
          }
      }
      for (; j < k; ++j)
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const f32x4_t v = on[u] ? __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(
                                        y + (t[u] * k + MOE_SLOT(j, k)) * d + col0 + col[u]))
                                  : f32x4_t{0.f, 0.f, 0.f, 0.f};
          const float wj = wts[(t0 + t[u]) * k + MOE_SLOT(j, k)];
          acc[u][0] = fmaf(wj, v[0], acc[u][0]);
          acc[u][1] = fmaf(wj, v[1], acc[u][1]);
          acc[u][2] = fmaf(wj, v[2], acc[u][2]);
          acc[u][3] = fmaf(wj, v[3], acc[u][3]);
        }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (!on[u]) continue;
        const int c = c0 + 64 * u;
        const f32x4_t sv = *reinterpret_cast<const f32x4_t*>(stg + (c / CPR) * NCOL + col[u]);
        const float a0 = routed_sum<T>(acc[u][0]) + sv[0], a1 = routed_sum<T>(acc[u][1]) + sv[1];
        const float a2 = routed_sum<T>(acc[u][2]) + sv[2], a3 = routed_sum<T>(acc[u][3]) + sv[3];
        T* o = out + (t0 + t[u]) * d + col0 + col[u];
        if constexpr (sizeof(T) == 2) {
          *reinterpret_cast<uint2*>(o) = uint2{f32x2_to_bf16x2(a0, a1), f32x2_to_bf16x2(a2, a3)};
        } else {
          *reinterpret_cast<f32x4_t*>(o) = f32x4_t{a0, a1, a2, a3};
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

struct DownParams {
  const void* h;          // [rows, K] intermediate
  int64_t n;              // dense: rows
  int d, K;               // output width, reduction size (I or I_s)
  const void* w;          // dense: [d, K]
  GemmGroups g;           // grouped: routed experts (down part of each line)
  int64_t line_down_off;  // grouped: element offset of W_down inside a line (2*I*d)
  const int32_t* row_slot;// grouped: output row (t*k + j) of each permuted row
  float* out;             // grouped: Y [n*k, d]; dense without cout: S [n, d]
  unsigned long long* clk;   // profiling clock counters of the stage, or NULL
  // dense (the shared expert), with the combine in the epilogue; S stays in registers:
  const float* y;         // Y [n*k, d], unweighted fp32 rows of the routed experts
  const float* wts;       // [T, k] slot weights, row t0 + t for chunk token t
  int64_t t0;             // first prompt row of the chunk
  int k;                  // slots per token
  void* cout;             // [T, d] layer output (dtype), rows t0 .. t0 + n - 1 written; NULL:
                          // the dense GEMM writes S to `out` instead
};

// Work units (M-tile x N-tile) of a down launch; a tile-list entry taller than this tile shape
// is worked as tile_rows / BM stacked tiles.
template <class TL, bool kGrouped>
__device__ __forceinline__ int down_units(const DownParams& p) {
  const int NT = (p.d + TL::BN - 1) / TL::BN;
  const int sub = kGrouped ? p.g.tile_rows / TL::BM : 1;
  const int m_tiles = kGrouped ? max(0, min(p.g.tile_cap, *p.g.n_mtiles - p.g.tile_lo)) * sub
                               : static_cast<int>((p.n + TL::BM - 1) / TL::BM);
  return m_tiles * NT;
}

template <typename T, class TL, bool kGrouped, bool kEarlySlots = kGrouped>
__device__ __forceinline__ void down_tile(const DownParams& p, int t, char* lds);

template <typename T, class TL, bool kGrouped>
__global__ __launch_bounds__(TL::NT) __attribute__((amdgpu_waves_per_eu(2)))
void down_kernel(DownParams p) {
  __shared__ __attribute__((aligned(1024))) char lds[TL::LDS];
  int t;
  if (!xcd_tile(down_units<TL, kGrouped>(p), &t)) return;
  down_tile<T, TL, kGrouped>(p, t, lds);
}

// The shared expert's down units (S alone) and the routed ones in one launch (shared units
// first), as gu_mixed_kernel does for the gate/up GEMMs: the same tiles, so the same bits.
template <typename T, class TL>
__global__ __launch_bounds__(TL::NT) __attribute__((amdgpu_waves_per_eu(2)))
void down_mixed_kernel(DownParams shared, DownParams routed) {
  __shared__ __attribute__((aligned(1024))) char lds[TL::LDS];
  const int ns = down_units<TL, false>(shared);
  int t;
  if (!xcd_tile(ns + down_units<TL, true>(routed), &t)) return;
  if (t < ns)
    down_tile<T, TL, false>(shared, t, lds);
  else
    down_tile<T, TL, true, false>(routed, t - ns, lds);
}

// The previous chunk's shared down GEMM with the combine in its epilogue (dense down units, as
// down_kernel works them) and this chunk's shared and routed gate/up units, in one launch: a
// layer call of several chunks defers each chunk's shared down + combine to the next chunk's
// gate/up launch, which does not depend on it. Alone, that GEMM gives the chip one tile per CU
// or less at 1,024 to 4,096 tokens a chunk; here its units run beside the gate/up units. Same
// tiles, instruction and K order as the stand-alone launch (row-invariant), so the same bits.
// On 64-row and decode tiles the down units start first on every XCD; on taller ones they come
// last and fill the gate/up launch's partial last round (each order measured faster on its
// tiles). On decode tiles (chunks of 193 to 512 tokens) the shared gate/up units are 16-row
// blocks too.
template <typename T, class TL>
__global__ __launch_bounds__(TL::NT) __attribute__((amdgpu_waves_per_eu(2)))
void gu_mixed_combine_kernel(DownParams prev, GuParams shared, GuParams routed) {
  __shared__ __attribute__((aligned(1024))) char lds[TL::LDS];
  constexpr bool kDownFirst = TL::BM <= SmallTile::BM;
  const int nd = prev.cout ? down_units<TL, false>(prev) : 0;
  const int ns = gu_units<TL, false>(shared);
  const int ng = ns + gu_units<TL, true>(routed);
  int t;
  bool in_a;
  if (!(kDownFirst ? xcd_tile_two(nd, ng, &t, &in_a) : xcd_tile_two(ng, nd, &t, &in_a))) return;
  if (in_a == kDownFirst)
    down_tile<T, TL, false>(prev, t, lds);
  else if (t < ns)
    gu_tile<T, TL, false>(shared, t, lds);
  else
    gu_tile<T, TL, true>(routed, t - ns, lds);
}

template <typename T, class TL, bool kGrouped, bool kEarlySlots>
__device__ __forceinline__ void down_tile(const DownParams& p, int t, char* lds) {
  const int NT = (p.d + TL::BN - 1) / TL::BN;
  const int sub = kGrouped ? p.g.tile_rows / TL::BM : 1;
  ClockSample clock(p.clk);
  const int mi = t / NT;
  const int n0 = (t % NT) * TL::BN;
  int64_t row0;
  int rows;
  const char* wbase;
  if (kGrouped) {
    const MTile mt = p.g.mtiles[p.g.tile_lo + mi / sub];
    const int m0 = mt.m0 + (mi % sub) * TL::BM;
    rows = min(TL::BM, p.g.counts[mt.group] - m0);
    if (rows <= 0) return;
    row0 = static_cast<int64_t>(p.g.offsets[mt.group]) + m0;
    const char* line = line_of(p.g, mt.group);
    wbase = line ? line + p.line_down_off * static_cast<int64_t>(sizeof(T)) : nullptr;
  } else {
    row0 = static_cast<int64_t>(mi) * TL::BM;
    rows = static_cast<int>(min<int64_t>(TL::BM, p.n - row0));
    wbase = static_cast<const char*>(p.w);
  }
  const bool missing = wbase == nullptr;
  const size_t rowb = static_cast<size_t>(p.K) * sizeof(T);
  const char* src[TL::LPW];
#pragma unroll
  for (int q = 0; q < TL::LPW; ++q) {
    const int r = stage_row<TL>(q);
    const char* base;
    if (r < TL::BM) {
      base = static_cast<const char*>(p.h) + (row0 + (r < rows ? r : 0)) * rowb;
    } else {
      const int wr = n0 + r - TL::BM;
      base = missing ? static_cast<const char*>(p.h)
                     : wbase + static_cast<int64_t>(wr < p.d ? wr : n0) * rowb;
    }
    src[q] = base + 16 * stage_seg<TL>();
  }
  // The output row (token slot) of each of the wave's rows, written to LDS beside the staging
  // area after the mainloop (the stage buffers hold that space until then). Looked up per
  // store instead, each lookup would wait on a global load, and that wait (vmcnt) also waits
  // for every store the wave has issued before it. With kEarlySlots the slots are loaded
  // before the mainloop, so their latency hides behind the first stage. Not in the launch that
  // also runs dense tiles (down_mixed_kernel): the compiler shares one stage loop between its
  // two tile kinds, and the early load's register, live into that loop, made it wait for every
  // stage load at each stage (the decode-sized down 30 -> 40 us).
  constexpr int kTab = TL::FM * 16;
  constexpr int kTabPerLane = (kTab + 63) / 64;
  int slot_of[kTabPerLane];
  auto load_slots = [&]() {
    const int lane = threadIdx.x & 63, wm = (threadIdx.x >> 6) / TL::WN;
#pragma unroll
    for (int q = 0; q < kTabPerLane; ++q) {
      const int idx = lane + 64 * q;
      const int tr = block_row<TL>(idx >> 4, wm) + (idx & 15);
      slot_of[q] = (idx < kTab && tr < rows) ? p.row_slot[row0 + tr] : -1;
    }
  };
  if constexpr (kGrouped && kEarlySlots) load_slots();
  f32x4_t acc[TL::FM][TL::FN];
  if (!missing)
    mainloop<T, TL, false>(src, stages<T, TL>(p.K), lds, acc, rows);

  const int wave = threadIdx.x >> 6;
  const int wm = wave / TL::WN, wn = wave % TL::WN;
  auto val = [&](int i, int j, int r) -> float {
    return missing ? __builtin_nanf("") : acc[i][j][r];
  };
  const int col0 = n0 + wn * TL::TN;
  if (kGrouped) {
    if constexpr (!kEarlySlots) load_slots();
    const int lane = threadIdx.x & 63;
    constexpr int kStage = 16 * TL::TN * static_cast<int>(sizeof(float)) * TL::NW;
    static_assert(kStage + TL::NW * kTab * 4 <= TL::LDS, "slot table fits in LDS");
    int* tab = reinterpret_cast<int*>(lds + kStage) + wave * kTab;
#pragma unroll
    for (int q = 0; q < kTabPerLane; ++q)
      if (lane + 64 * q < kTab) tab[lane + 64 * q] = slot_of[q];
    __builtin_amdgcn_wave_barrier();  // a wave's LDS writes land before its later LDS reads
    auto row_of = [&](int sr) -> int64_t { return tab[sr]; };   // sr = block * 16 + row
    store_slab<TL, float, TL::TN, true>(lds, val, row_of, p.out, p.d, col0, min(TL::TN, p.d - col0));
  } else if (p.cout) {
    combine_slab<TL, T>(lds, val, wm, row0, rows, p.y, p.wts, p.t0, p.k, p.d,
                        static_cast<T*>(p.cout), col0, min(TL::TN, p.d - col0));
  } else {                      // the shared expert's S alone (fp32), for the stand-alone combine
    auto row_of = [&](int sr) -> int64_t {
      const int tr = block_row<TL>(sr >> 4, wm) + (sr & 15);
      return tr < rows ? row0 + tr : -1;
    };
    store_slab<TL, float, TL::TN>(lds, val, row_of, p.out, p.d, col0, min(TL::TN, p.d - col0));
  }
  clock.finish();
}

// ---------------------------------------------------------------- fused gate/up -> down
// One workgroup per routed M-tile of at most 64 rows (the small tile's height) runs both of the
// tile's GEMMs, and h never leaves the CU:
//   1. gate/up over I / 128 N-chunks, each with the small tile's mainloop (the same loads,
//      instruction, K order and lane mapping as the separate gate/up launch), its epilogue
//      writing silu(gate) * up, rounded to bf16, into an LDS copy of the tile's h rows;
//   2. down over the d / 256 N-chunks, the weight rows staged through two LDS buffers in one
//      pipeline across the chunks and h read from LDS as the A operand, in the K order and lane
//      mapping of the separate down launch; each chunk's Y goes out as there.
// So h and Y are bit for bit those of the two launches. One pipeline carried through both steps
// (no refill between the gate/up chunks) measured 3% slower than this with per-block fragment
// reads, and 10-12% slower with all of a K step's fragments read before its MFMAs. LDS: the
// small tile's 80 KB of stage buffers (in step 2 two 32 KB weight stages and the 16 KB output
// staging), then h (64 rows x I bf16, I <= 512), then the output-slot table.
using FusedTile = SmallTile;
constexpr int kFusedMaxI = 512;
constexpr int kFusedHOff = FusedTile::LDS;
constexpr int kFusedTabOff = kFusedHOff + FusedTile::BM * kFusedMaxI * 2;
constexpr int kFusedLds = kFusedTabOff + FusedTile::NW * FusedTile::FM * 16 * 4;
constexpr int kFusedBStage = FusedTile::BN * FusedTile::RB;        // 256 weight rows x 128 B
static_assert(2 * kFusedBStage + 16 * FusedTile::TN * 4 * FusedTile::NW <= FusedTile::LDS,
              "two weight stages and the output staging fit in the stage buffers");
static_assert(kFusedLds <= 160 * 1024, "LDS of one CU");

struct FusedParams {
  GuParams gu;            // prompt rows, d, I, groups, row_tok (gu.h unused)
  int64_t line_down_off;  // element offset of W_down inside a line (2*I*d)
  const int32_t* row_slot;
  float* y;               // Y [n*k, d]
};

// Byte offset of h element (r, c) in the LDS copy: row r holds I bf16 in 128-byte K stages,
// 16-byte segment g of a stage at g ^ (r & 7), the swizzle of the staged operand rows.
__device__ __forceinline__ int fused_h_off(int r, int c, int I) {
  return r * I * 2 + (c >> 6) * 128 + ((((c >> 3) & 7) ^ (r & 7)) << 4) + (c & 7) * 2;
}

__global__ __launch_bounds__(FusedTile::NT)
void gu_down_fused_kernel(FusedParams p) {
  using TL = FusedTile;
  using T = uint16_t;
  using F = Frag<T>;
  __shared__ __attribute__((aligned(1024))) char lds[kFusedLds];
  const GuParams& q = p.gu;
  const int m_tiles = max(0, min(q.g.tile_cap, *q.g.n_mtiles - q.g.tile_lo));
  int t;
  if (!xcd_tile(m_tiles, &t)) return;
  ClockSample clock(q.clk);
  const MTile mt = q.g.mtiles[q.g.tile_lo + t];
  const int64_t row0 = static_cast<int64_t>(q.g.offsets[mt.group]) + mt.m0;
  const int rows = min(TL::BM, q.g.counts[mt.group] - mt.m0);
  const char* line = line_of(q.g, mt.group);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wn = wave % TL::WN, kq = lane >> 4, l16 = lane & 15;
  const int I = q.I, d = q.d;
  char* hl = lds + kFusedHOff;

  // output slot of each tile row, one copy per wave (read before any store needs it)
  int* tab = reinterpret_cast<int*>(lds + kFusedTabOff) + wave * (TL::FM * 16);
  for (int idx = lane; idx < TL::FM * 16; idx += 64)
    tab[idx] = idx < rows ? p.row_slot[row0 + idx] : -1;
  __builtin_amdgcn_wave_barrier();
  auto row_of = [&](int sr) -> int64_t { return tab[sr]; };     // sr = block * 16 + row
  auto store_y = [&](auto val, int c) {
    const int col0 = c * TL::BN + wn * TL::TN;
    store_slab<TL, float, TL::TN, true>(lds + 2 * kFusedBStage, val, row_of, p.y, d, col0,
                                        min(TL::TN, d - col0));
  };
  const int n_dc = (d + TL::BN - 1) / TL::BN;
  if (line == nullptr) {        // offloaded expert that was not staged: its Y rows are NaN
    for (int c = 0; c < n_dc; ++c)
      store_y([&](int, int, int) { return __builtin_nanf(""); }, c);
    clock.finish();
    return;
  }

  // 1. gate/up, h into LDS
  constexpr int HC = TL::BN / 2;
  const size_t rowb = static_cast<size_t>(d) * sizeof(T);
  f32x4_t acc[TL::FM][TL::FN];
  for (int n0h = 0; n0h < I; n0h += HC) {
    const char* src[TL::LPW];
#pragma unroll
    for (int qq = 0; qq < TL::LPW; ++qq) {
      const int r = stage_row<TL>(qq);
      const char* base;
      if (r < TL::BM) {
        const int ar = r < rows ? r : 0;
        base = static_cast<const char*>(q.x) + (q.t0 + q.row_tok[row0 + ar]) * rowb;
      } else {
        const int br = r - TL::BM;
        const int hc = n0h + (br < HC ? br : br - HC);
        base = line + static_cast<int64_t>((hc < I ? hc : n0h) + (br < HC ? 0 : I)) * rowb;
      }
      src[qq] = base + 16 * stage_seg<TL>();
    }
    mainloop<T, TL, true>(src, stages<T, TL>(d), lds, acc, rows);
    constexpr int H = TL::FN / 2;
#pragma unroll
    for (int i = 0; i < TL::FM; ++i)
#pragma unroll
      for (int j = 0; j < H; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = block_row<TL>(i, 0) + 4 * kq + r;
          const int col = n0h + wn * (TL::TN / 2) + j * 16 + l16;
          *reinterpret_cast<T*>(hl + fused_h_off(row, col, I)) =
              h_store<T>(silu_f32(acc[i][j][r]) * acc[i][j + H][r]);
        }
  }
  __syncthreads();              // h complete; the stage buffers are free

  // 2. down: weight rows of N-chunk c, K stage s, through buffer (c * nk + s) % 2
  const int nk = stages<T, TL>(I);
  const int G = n_dc * nk;
  const char* wdown = line + p.line_down_off * static_cast<int64_t>(sizeof(T));
  const size_t rowk = static_cast<size_t>(I) * sizeof(T);
  constexpr int LPB = kFusedBStage / 1024 / TL::NW;     // load instructions per wave and stage
  typedef __attribute__((address_space(3))) char lds_char;
  const uint32_t wave_lds = __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>((uintptr_t)(lds_char*)lds) + static_cast<uint32_t>(wave * 1024));
  const int seg16 = 16 * stage_seg<TL>();
  auto issue_b = [&](int g) {
    const int c = g / nk, ko = (g % nk) * TL::RB;
    const uint32_t dst = wave_lds + static_cast<uint32_t>((g & 1) * kFusedBStage);
#pragma unroll
    for (int qq = 0; qq < LPB; ++qq) {
      const int wr = c * TL::BN + (wave + TL::NW * qq) * TL::RPL + lane / TL::SPR;
      const char* src = wdown + static_cast<int64_t>(wr < d ? wr : c * TL::BN) * rowk + ko + seg16;
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
      asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
                   :
                   : "s"(__builtin_amdgcn_readfirstlane(dst + static_cast<uint32_t>(qq * TL::NW * 1024))),
                     "v"(src)
                   : "memory", "m0");
#pragma clang diagnostic pop
    }
  };
  const int sw = swz<TL>(l16);
  int hrow[TL::FM], brow[TL::FN];
#pragma unroll
  for (int i = 0; i < TL::FM; ++i) hrow[i] = (block_row<TL>(i, 0) + l16) * I * 2;
#pragma unroll
  for (int j = 0; j < TL::FN; ++j) brow[j] = (wn * TL::TN + j * 16 + l16) * TL::RB;
  const int nbusy = busy_blocks<TL>(rows, 0);
#pragma unroll
  for (int i = 0; i < TL::FM; ++i)
#pragma unroll
    for (int j = 0; j < TL::FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  issue_b(0);
  for (int g = 0; g < G; ++g) {
    wait_vmcnt<0>();            // this wave's share of stage g (and earlier Y stores) landed
    __syncthreads();            // everyone's; everyone also left stage g - 1
    if (g + 1 < G) issue_b(g + 1);
    const int s = g % nk;
    const char* bbuf = lds + (g & 1) * kFusedBStage;
    const char* hbase = hl + s * TL::RB;
    constexpr int kSteps = TL::RB / F::kStepBytes;
#pragma unroll
    for (int ks = 0; ks < kSteps; ++ks) {
      typename F::V b[TL::FN];
#pragma unroll
      for (int j = 0; j < TL::FN; ++j) b[j] = F::load(bbuf + brow[j], ks, kq, sw);
#pragma unroll
      for (int i = 0; i < TL::FM; ++i) {
        if (i < nbusy) {
          const typename F::V a = F::load(hbase + hrow[i], ks, kq, sw);
#pragma unroll
          for (int j = 0; j < TL::FN; ++j) acc[i][j] = F::mma(a, b[j], acc[i][j]);
        }
      }
    }
    if (s == nk - 1) {          // chunk done: its Y rows out, accumulators reset
      store_y([&](int i, int j, int r) { return acc[i][j][r]; }, g / nk);
#pragma unroll
      for (int i = 0; i < TL::FM; ++i)
#pragma unroll
        for (int j = 0; j < TL::FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  }
  clock.finish();
}

struct RouterParams {
  const void* x;
  const void* w;
  const float* bias;
  float* logits;
  int64_t T;
  int d, E;
  unsigned long long* clk;   // profiling clock counters of the stage, or NULL
};

template <typename T, class TL>
__global__ __launch_bounds__(TL::NT) __attribute__((amdgpu_waves_per_eu(2)))
void router_kernel(RouterParams p) {
  __shared__ __attribute__((aligned(1024))) char lds[TL::LDS];
  const int NT = (p.E + TL::BN - 1) / TL::BN;
  int t;
  if (!xcd_tile(static_cast<int>((p.T + TL::BM - 1) / TL::BM) * NT, &t)) return;
  ClockSample clock(p.clk);
  const int n0 = (t % NT) * TL::BN;
  const int64_t row0 = static_cast<int64_t>(t / NT) * TL::BM;
  const int rows = static_cast<int>(min<int64_t>(TL::BM, p.T - row0));
  const size_t rowb = static_cast<size_t>(p.d) * sizeof(T);
  const char* src[TL::LPW];
#pragma unroll
  for (int q = 0; q < TL::LPW; ++q) {
    const int r = stage_row<TL>(q);
    const char* base;
    if (r < TL::BM) {
      base = static_cast<const char*>(p.x) + (row0 + (r < rows ? r : 0)) * rowb;
    } else {
      const int wr = n0 + r - TL::BM;
      base = static_cast<const char*>(p.w) + static_cast<int64_t>(wr < p.E ? wr : n0) * rowb;
    }
    src[q] = base + 16 * stage_seg<TL>();
  }
  f32x4_t acc[TL::FM][TL::FN];
  mainloop<T, TL, false>(src, stages<T, TL>(p.d), lds, acc, rows);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / TL::WN, wn = wave % TL::WN;
  const int col0 = n0 + wn * TL::TN;
  auto val = [&](int i, int j, int r) -> float {
    const int col = col0 + j * 16 + (lane & 15);
    return acc[i][j][r] + ((p.bias && col < p.E) ? p.bias[col] : 0.0f);
  };
  auto row_of = [&](int sr) -> int64_t {      // sr = block * 16 + row in block
    const int tr = block_row<TL>(sr >> 4, wm) + (sr & 15);
    return tr < rows ? row0 + tr : -1;
  };
  store_slab<TL, float, TL::TN>(lds, val, row_of, p.logits, p.E, col0, min(TL::TN, p.E - col0));
  clock.finish();
}

constexpr int64_t kCus = 256;      // compute units of an MI355X

// Dense GEMMs (router, shared expert): big tiles when they still give the chip about two
// workgroups per CU (384 of them: 1.5 per CU), else 128-row tiles while they give 0.75 per CU
// (at 2,048 or 4,096 rows a chunk, the 64-row tiles would re-read the shared weights 32 or 64
// times), else small ones: with four stage buffers when there is at most one per CU, so the
// few tiles keep three K stages in flight instead of one, and half as wide when there would be
// at most half a tile per CU (twice the tiles; in the shared down each then combines half the
// columns). The shared expert's GEMMs of at most 512 rows take narrower tiles ahead of these
// (decode tiles up to 64 rows, then 64x64).
inline bool use_big_dense(int64_t n, int64_t n_tiles_big) {
  return n >= BigTile::BM && ((n + BigTile::BM - 1) / BigTile::BM) * n_tiles_big >= 384;
}

}  // namespace

int routed_tile_rows(int64_t n, int k, int E) {
  // a = mean rows per expert. With a in [192, 320) many experts hold just over 256 rows; a
  // 320-row tile keeps them in one tile instead of a full tile plus a nearly empty one. With
  // a in [48, 128), 128-row tiles do the same for experts just over 64 rows: an expert's
  // second M-tile would stream its weight slice again (the MFMAs of empty row blocks are
  // skipped either way).
  const int64_t rows = n * k, e = static_cast<int64_t>(E);
  if (rows < e * 16) return DecodeTile::BM;
  if (rows >= e * 192 && rows < e * 320) return TallTile::BM;
  if (rows >= e * 48 && rows < e * 128) return MidTile::BM;
  return rows >= e * 128 ? BigTile::BM : SmallTile::BM;
}

hipError_t launch_router_gemm(int dtype, const void* x, const void* w_router, const float* bias,
                              int64_t T, int d, int E, float* logits, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  ProfScope prof(MOE_STAGE_ROUTER, s);
  RouterParams p{x, w_router, bias, logits, T, d, E, prof_clock(MOE_STAGE_ROUTER)};
  const int64_t mid_tiles = (T + MidTile::BM - 1) / MidTile::BM * ((E + MidTile::BN - 1) / MidTile::BN);
  const int64_t t16 = (T + RouterTile16::BM - 1) / RouterTile16::BM *
                      ((E + RouterTile16::BN - 1) / RouterTile16::BN);
  const int64_t t64 = (T + RouterTile64::BM - 1) / RouterTile64::BM *
                      ((E + RouterTile64::BN - 1) / RouterTile64::BN);
  if (T <= RouterTile16::BM || t16 <= 128) {
    const unsigned grid = xcd_grid(t16);
    if (dtype == MOE_BF16) router_kernel<uint16_t, RouterTile16><<<grid, RouterTile16::NT, 0, s>>>(p);
    else router_kernel<float, RouterTile16><<<grid, RouterTile16::NT, 0, s>>>(p);
  } else if (use_big_dense(T, (E + BigTile::BN - 1) / BigTile::BN)) {
    const unsigned grid = xcd_grid((T + BigTile::BM - 1) / BigTile::BM * ((E + BigTile::BN - 1) / BigTile::BN));
    if (dtype == MOE_BF16) router_kernel<uint16_t, BigTile><<<grid, BigTile::NT, 0, s>>>(p);
    else router_kernel<float, BigTile><<<grid, BigTile::NT, 0, s>>>(p);
  } else if (mid_tiles >= 192) {
    // 128-row tiles while they still give 0.75 tiles per CU: the two halves share each staged
    // weight row (a third fewer stage bytes than two 64-row tiles) -- 55 against 63 us for the
    // 16,022 x 2,048 x 512 router
    const unsigned grid = xcd_grid(mid_tiles);
    if (dtype == MOE_BF16) router_kernel<uint16_t, MidTile><<<grid, MidTile::NT, 0, s>>>(p);
    else router_kernel<float, MidTile><<<grid, MidTile::NT, 0, s>>>(p);
  } else if (t64 <= 512) {
    const unsigned grid = xcd_grid(t64);
    if (dtype == MOE_BF16) router_kernel<uint16_t, RouterTile64><<<grid, RouterTile64::NT, 0, s>>>(p);
    else router_kernel<float, RouterTile64><<<grid, RouterTile64::NT, 0, s>>>(p);
  } else if (const int64_t st = (T + SmallTile::BM - 1) / SmallTile::BM * ((E + SmallTile::BN - 1) / SmallTile::BN);
             st <= kCus) {
    const unsigned grid = xcd_grid(st);
    if (dtype == MOE_BF16) router_kernel<uint16_t, SmallTile4><<<grid, SmallTile4::NT, 0, s>>>(p);
    else router_kernel<float, SmallTile4><<<grid, SmallTile4::NT, 0, s>>>(p);
  } else {
    const unsigned grid = xcd_grid((T + SmallTile::BM - 1) / SmallTile::BM * ((E + SmallTile::BN - 1) / SmallTile::BN));
    if (dtype == MOE_BF16) router_kernel<uint16_t, SmallTile><<<grid, SmallTile::NT, 0, s>>>(p);
    else router_kernel<float, SmallTile><<<grid, SmallTile::NT, 0, s>>>(p);
  }
  return hipGetLastError();
}

template <class TL>
static void gu_routed(int dtype, const GuParams& p, const GemmGroups& g, int I, hipStream_t s) {
  const unsigned grid = xcd_grid(static_cast<int64_t>(g.tile_cap) * ((I + TL::BN / 2 - 1) / (TL::BN / 2)));
  if (dtype == MOE_BF16) gu_kernel<uint16_t, TL, true><<<grid, TL::NT, 0, s>>>(p);
  else gu_kernel<float, TL, true><<<grid, TL::NT, 0, s>>>(p);
}

hipError_t launch_gu_routed(int dtype, const void* x, int64_t t0, int d, int I,
                            const GemmGroups& g, const int32_t* row_tok, void* h, hipStream_t s) {
  if (g.tile_cap <= 0) return hipSuccess;
  ProfScope prof(MOE_STAGE_GU_ROUTED, s);
  GuParams p{};
  p.x = x; p.t0 = t0; p.n = 0; p.d = d; p.I = I; p.w = nullptr; p.g = g;
  p.row_tok = row_tok; p.h = h; p.clk = prof_clock(MOE_STAGE_GU_ROUTED);
  if (g.tile_rows == TallTile::BM) gu_routed<TallTile>(dtype, p, g, I, s);
  else if (g.tile_rows == BigTile::BM) gu_routed<BigTile>(dtype, p, g, I, s);
  else if (g.tile_rows == MidTile::BM) gu_routed<MidTile>(dtype, p, g, I, s);
  else if (g.tile_rows == DecodeTile::BM) gu_routed<DecodeTile>(dtype, p, g, I, s);
  else gu_routed<SmallTile>(dtype, p, g, I, s);
  return hipGetLastError();
}

template <class TL>
static void gu_mixed(int dtype, const GuParams& ps, const GuParams& pr, hipStream_t s) {
  constexpr int HC = TL::BN / 2;
  const int64_t units = (ps.n + TL::BM - 1) / TL::BM * ((ps.I + HC - 1) / HC) +
                        static_cast<int64_t>(pr.g.tile_cap) * ((pr.I + HC - 1) / HC);
  const unsigned grid = xcd_grid(units);
  if (dtype == MOE_BF16) gu_mixed_kernel<uint16_t, TL><<<grid, TL::NT, 0, s>>>(ps, pr);
  else gu_mixed_kernel<float, TL><<<grid, TL::NT, 0, s>>>(ps, pr);
}

bool gu_mixed_supported(int tile_rows, int64_t n) {
  return tile_rows == TallTile::BM || tile_rows == BigTile::BM || tile_rows == MidTile::BM ||
         (tile_rows == SmallTile::BM && n > DecodeTile::BM) ||
         (tile_rows == DecodeTile::BM && n <= kMixedDecodeRows);
}

hipError_t launch_gu_mixed(int dtype, const void* x, int64_t t0, int64_t n, int d, int I, int Is,
                           const void* w_gu_shared, void* h_shared, const GemmGroups& g,
                           const int32_t* row_tok, void* h, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  ProfScope prof(MOE_STAGE_GU_MIXED, s);
  GuParams ps{}, pr{};
  ps.x = x; ps.t0 = t0; ps.n = n; ps.d = d; ps.I = Is; ps.w = w_gu_shared; ps.h = h_shared;
  ps.clk = prof_clock(MOE_STAGE_GU_MIXED);
  pr.x = x; pr.t0 = t0; pr.n = 0; pr.d = d; pr.I = I; pr.w = nullptr; pr.g = g;
  pr.row_tok = row_tok; pr.h = h; pr.clk = ps.clk;
  if (g.tile_rows == TallTile::BM) gu_mixed<TallTile>(dtype, ps, pr, s);
  else if (g.tile_rows == BigTile::BM) gu_mixed<BigTile>(dtype, ps, pr, s);
  else if (g.tile_rows == MidTile::BM) gu_mixed<MidTile>(dtype, ps, pr, s);
  else if (g.tile_rows == SmallTile::BM && n > DecodeTile::BM) gu_mixed<SmallTile>(dtype, ps, pr, s);
  else if (g.tile_rows == DecodeTile::BM && n <= kMixedDecodeRows) gu_mixed<DecodeTile>(dtype, ps, pr, s);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

template <class TL>
static void gu_mixed_combine(int dtype, const DownParams& pd, const GuParams& ps,
                             const GuParams& pr, hipStream_t s) {
  constexpr int HC = TL::BN / 2;
  const int64_t nd = pd.cout ? (pd.n + TL::BM - 1) / TL::BM * ((pd.d + TL::BN - 1) / TL::BN) : 0;
  const int64_t ng = (ps.n + TL::BM - 1) / TL::BM * ((ps.I + HC - 1) / HC) +
                     static_cast<int64_t>(pr.g.tile_cap) * ((pr.I + HC - 1) / HC);
  const unsigned grid = xcd_grid(nd) + xcd_grid(ng);
  if (dtype == MOE_BF16) gu_mixed_combine_kernel<uint16_t, TL><<<grid, TL::NT, 0, s>>>(pd, ps, pr);
  else gu_mixed_combine_kernel<float, TL><<<grid, TL::NT, 0, s>>>(pd, ps, pr);
}

bool gu_mixed_combine_supported(int tile_rows, int64_t n) {
  return tile_rows == BigTile::BM || tile_rows == MidTile::BM ||
         (tile_rows == SmallTile::BM && n > DecodeTile::BM) ||
         (tile_rows == DecodeTile::BM && n > kMixedDecodeRows && n <= kDeferDecodeRows);
}

hipError_t launch_gu_mixed_combine(int dtype, const void* x, int64_t t0, int64_t n, int d, int I,
                                   int Is, const void* w_gu_shared, void* h_shared,
                                   const GemmGroups& g, const int32_t* row_tok, void* h,
                                   const void* prev_h_shared, int64_t prev_t0, int64_t prev_n,
                                   const void* w_down_shared, const float* y,
                                   const float* weights, int k, void* out, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (!gu_mixed_combine_supported(g.tile_rows, n)) return hipErrorInvalidValue;
  ProfScope prof(MOE_STAGE_GU_MIXED, s);
  GuParams ps{}, pr{};
  ps.x = x; ps.t0 = t0; ps.n = n; ps.d = d; ps.I = Is; ps.w = w_gu_shared; ps.h = h_shared;
  ps.clk = prof_clock(MOE_STAGE_GU_MIXED);
  pr.x = x; pr.t0 = t0; pr.n = 0; pr.d = d; pr.I = I; pr.w = nullptr; pr.g = g;
  pr.row_tok = row_tok; pr.h = h; pr.clk = ps.clk;
  DownParams pd{};
  pd.h = prev_h_shared; pd.n = prev_n; pd.d = d; pd.K = Is; pd.w = w_down_shared;
  pd.line_down_off = 0; pd.row_slot = nullptr; pd.out = nullptr; pd.clk = ps.clk;
  pd.y = y; pd.wts = weights; pd.t0 = prev_t0; pd.k = k;
  pd.cout = prev_n > 0 ? out : nullptr;
  if (g.tile_rows == BigTile::BM) gu_mixed_combine<BigTile>(dtype, pd, ps, pr, s);
  else if (g.tile_rows == MidTile::BM) gu_mixed_combine<MidTile>(dtype, pd, ps, pr, s);
  else if (g.tile_rows == DecodeTile::BM) gu_mixed_combine<DecodeTile>(dtype, pd, ps, pr, s);
  else gu_mixed_combine<SmallTile>(dtype, pd, ps, pr, s);
  return hipGetLastError();
}

hipError_t launch_down_mixed(int dtype, const void* h_shared, int64_t n, int d, int Is,
                             const void* w_down_shared, float* s_out, const void* h, int I,
                             const GemmGroups& g, const int32_t* row_slot, float* y,
                             hipStream_t s) {
  using TL = DecodeTile;
  if (n <= 0) return hipSuccess;
  if (g.tile_rows != TL::BM || n > kMixedDecodeRows) return hipErrorInvalidValue;
  ProfScope prof(MOE_STAGE_DOWN_MIXED, s);
  DownParams ps{}, pr{};
  ps.h = h_shared; ps.n = n; ps.d = d; ps.K = Is; ps.w = w_down_shared; ps.out = s_out;
  ps.clk = prof_clock(MOE_STAGE_DOWN_MIXED);
  pr.h = h; pr.n = 0; pr.d = d; pr.K = I; pr.w = nullptr; pr.g = g;
  pr.line_down_off = 2LL * I * d; pr.row_slot = row_slot; pr.out = y; pr.clk = ps.clk;
  const int64_t nt = (d + TL::BN - 1) / TL::BN;
  const unsigned grid = xcd_grid((n + TL::BM - 1) / TL::BM * nt + static_cast<int64_t>(g.tile_cap) * nt);
  if (dtype == MOE_BF16) down_mixed_kernel<uint16_t, TL><<<grid, TL::NT, 0, s>>>(ps, pr);
  else down_mixed_kernel<float, TL><<<grid, TL::NT, 0, s>>>(ps, pr);
  return hipGetLastError();
}

hipError_t launch_gu_dense(int dtype, const void* x, int64_t t0, int64_t n, int d, int Is,
                           const void* w_gu, void* h, hipStream_t s) {
  if (n <= 0 || Is <= 0) return hipSuccess;
  ProfScope prof(MOE_STAGE_GU_SHARED, s);
  GuParams p{};
  p.x = x; p.t0 = t0; p.n = n; p.d = d; p.I = Is; p.w = w_gu; p.row_tok = nullptr; p.h = h;
  p.clk = prof_clock(MOE_STAGE_GU_SHARED);
  const int64_t nt_big = (Is + BigTile::BN / 2 - 1) / (BigTile::BN / 2);
  if (n <= 4 * DecodeTile::BM) {
    const unsigned grid = xcd_grid((n + DecodeTile::BM - 1) / DecodeTile::BM *
                                   ((Is + DecodeTile::BN / 2 - 1) / (DecodeTile::BN / 2)));
    if (dtype == MOE_BF16) gu_kernel<uint16_t, DecodeTile, false><<<grid, DecodeTile::NT, 0, s>>>(p);
    else gu_kernel<float, DecodeTile, false><<<grid, DecodeTile::NT, 0, s>>>(p);
  } else if (n <= 8 * PairTile64::BM) {
    const unsigned grid = xcd_grid((n + PairTile64::BM - 1) / PairTile64::BM *
                                   ((Is + PairTile64::BN / 2 - 1) / (PairTile64::BN / 2)));
    if (dtype == MOE_BF16) gu_kernel<uint16_t, PairTile64, false><<<grid, PairTile64::NT, 0, s>>>(p);
    else gu_kernel<float, PairTile64, false><<<grid, PairTile64::NT, 0, s>>>(p);
  } else if (use_big_dense(n, nt_big)) {
    const unsigned grid = xcd_grid((n + BigTile::BM - 1) / BigTile::BM * nt_big);
    if (dtype == MOE_BF16) gu_kernel<uint16_t, BigTile, false><<<grid, BigTile::NT, 0, s>>>(p);
    else gu_kernel<float, BigTile, false><<<grid, BigTile::NT, 0, s>>>(p);
  } else if (const int64_t mt = (n + MidTile::BM - 1) / MidTile::BM *
                                ((Is + MidTile::BN / 2 - 1) / (MidTile::BN / 2));
             n >= MidTile::BM && mt >= 192) {
    const unsigned grid = xcd_grid(mt);
    if (dtype == MOE_BF16) gu_kernel<uint16_t, MidTile, false><<<grid, MidTile::NT, 0, s>>>(p);
    else gu_kernel<float, MidTile, false><<<grid, MidTile::NT, 0, s>>>(p);
  } else if (const int64_t st = (n + SmallTile::BM - 1) / SmallTile::BM *
                                ((Is + SmallTile::BN / 2 - 1) / (SmallTile::BN / 2));
             st <= kCus / 2) {
    const unsigned grid = xcd_grid((n + NarrowTile4::BM - 1) / NarrowTile4::BM *
                                   ((Is + NarrowTile4::BN / 2 - 1) / (NarrowTile4::BN / 2)));
    if (dtype == MOE_BF16) gu_kernel<uint16_t, NarrowTile4, false><<<grid, NarrowTile4::NT, 0, s>>>(p);
    else gu_kernel<float, NarrowTile4, false><<<grid, NarrowTile4::NT, 0, s>>>(p);
  } else if (const int64_t st = (n + SmallTile::BM - 1) / SmallTile::BM *
                                ((Is + SmallTile::BN / 2 - 1) / (SmallTile::BN / 2));
             st <= kCus) {
    const unsigned grid = xcd_grid(st);
    if (dtype == MOE_BF16) gu_kernel<uint16_t, SmallTile4, false><<<grid, SmallTile4::NT, 0, s>>>(p);
    else gu_kernel<float, SmallTile4, false><<<grid, SmallTile4::NT, 0, s>>>(p);
  } else {
    const unsigned grid = xcd_grid((n + SmallTile::BM - 1) / SmallTile::BM *
                                   ((Is + SmallTile::BN / 2 - 1) / (SmallTile::BN / 2)));
    if (dtype == MOE_BF16) gu_kernel<uint16_t, SmallTile, false><<<grid, SmallTile::NT, 0, s>>>(p);
    else gu_kernel<float, SmallTile, false><<<grid, SmallTile::NT, 0, s>>>(p);
  }
  return hipGetLastError();
}

template <class TL>
static void down_routed(int dtype, const DownParams& p, const GemmGroups& g, int d, hipStream_t s) {
  const unsigned grid = xcd_grid(static_cast<int64_t>(g.tile_cap) * (g.tile_rows / TL::BM) *
                                 ((d + TL::BN - 1) / TL::BN));
  if (dtype == MOE_BF16) down_kernel<uint16_t, TL, true><<<grid, TL::NT, 0, s>>>(p);
  else down_kernel<float, TL, true><<<grid, TL::NT, 0, s>>>(p);
}

hipError_t launch_down_routed(int dtype, const void* h, int d, int I, const GemmGroups& g,
                              const int32_t* row_slot, float* y, hipStream_t s) {
  if (g.tile_cap <= 0) return hipSuccess;
  ProfScope prof(MOE_STAGE_DOWN_ROUTED, s);
  DownParams p{};
  p.h = h; p.n = 0; p.d = d; p.K = I; p.w = nullptr; p.g = g;
  p.line_down_off = 2LL * I * d; p.row_slot = row_slot; p.out = y;
  p.clk = prof_clock(MOE_STAGE_DOWN_ROUTED);
  if (g.tile_rows == TallTile::BM) down_routed<TallTile>(dtype, p, g, d, s);
  else if (g.tile_rows == BigTile::BM) down_routed<BigTile>(dtype, p, g, d, s);
  else if (g.tile_rows == MidTile::BM) down_routed<MidTile>(dtype, p, g, d, s);
  else if (g.tile_rows == DecodeTile::BM) down_routed<DecodeTile>(dtype, p, g, d, s);
  else down_routed<SmallTile>(dtype, p, g, d, s);
  return hipGetLastError();
}

bool gu_down_fused_supported(int dtype, int tile_rows, int I) {
  return dtype == MOE_BF16 && tile_rows == FusedTile::BM && I > 0 && I <= kFusedMaxI &&
         I % (FusedTile::BN / 2) == 0;
}

hipError_t launch_gu_down_fused(const void* x, int64_t t0, int d, int I, const GemmGroups& g,
                                const int32_t* row_tok, const int32_t* row_slot, float* y,
                                hipStream_t s) {
  if (g.tile_cap <= 0) return hipSuccess;
  ProfScope prof(MOE_STAGE_GU_DOWN_FUSED, s);
  FusedParams p{};
  p.gu.x = x; p.gu.t0 = t0; p.gu.n = 0; p.gu.d = d; p.gu.I = I; p.gu.w = nullptr; p.gu.g = g;
  p.gu.row_tok = row_tok; p.gu.h = nullptr; p.gu.clk = prof_clock(MOE_STAGE_GU_DOWN_FUSED);
  p.line_down_off = 2LL * I * d; p.row_slot = row_slot; p.y = y;
  gu_down_fused_kernel<<<xcd_grid(g.tile_cap), FusedTile::NT, 0, s>>>(p);
  return hipGetLastError();
}

// Tile choice of the dense (shared-expert) down GEMM, with or without the combine.
static void down_dense(int dtype, const DownParams& p, int64_t n, int d, hipStream_t s) {
  const int64_t nt_big = (d + BigTile::BN - 1) / BigTile::BN;
  if (n <= 4 * DecodeTile::BM) {
    const unsigned grid = xcd_grid((n + DecodeTile::BM - 1) / DecodeTile::BM *
                                   ((d + DecodeTile::BN - 1) / DecodeTile::BN));
    if (dtype == MOE_BF16) down_kernel<uint16_t, DecodeTile, false><<<grid, DecodeTile::NT, 0, s>>>(p);
    else down_kernel<float, DecodeTile, false><<<grid, DecodeTile::NT, 0, s>>>(p);
  } else if (n <= 8 * RouterTile64::BM) {
    const unsigned grid = xcd_grid((n + RouterTile64::BM - 1) / RouterTile64::BM *
                                   ((d + RouterTile64::BN - 1) / RouterTile64::BN));
    if (dtype == MOE_BF16) down_kernel<uint16_t, RouterTile64, false><<<grid, RouterTile64::NT, 0, s>>>(p);
    else down_kernel<float, RouterTile64, false><<<grid, RouterTile64::NT, 0, s>>>(p);
  } else if (use_big_dense(n, nt_big)) {
    const unsigned grid = xcd_grid((n + BigTile::BM - 1) / BigTile::BM * nt_big);
    if (dtype == MOE_BF16) down_kernel<uint16_t, BigTile, false><<<grid, BigTile::NT, 0, s>>>(p);
    else down_kernel<float, BigTile, false><<<grid, BigTile::NT, 0, s>>>(p);
  } else if (const int64_t mt = (n + MidTile::BM - 1) / MidTile::BM *
                                ((d + MidTile::BN - 1) / MidTile::BN);
             n >= MidTile::BM && mt >= 192) {
    const unsigned grid = xcd_grid(mt);
    if (dtype == MOE_BF16) down_kernel<uint16_t, MidTile, false><<<grid, MidTile::NT, 0, s>>>(p);
    else down_kernel<float, MidTile, false><<<grid, MidTile::NT, 0, s>>>(p);
  } else if (const int64_t st = (n + SmallTile::BM - 1) / SmallTile::BM *
                                ((d + SmallTile::BN - 1) / SmallTile::BN);
             st <= kCus / 2) {
    const unsigned grid = xcd_grid((n + NarrowTile4::BM - 1) / NarrowTile4::BM *
                                   ((d + NarrowTile4::BN - 1) / NarrowTile4::BN));
    if (dtype == MOE_BF16) down_kernel<uint16_t, NarrowTile4, false><<<grid, NarrowTile4::NT, 0, s>>>(p);
    else down_kernel<float, NarrowTile4, false><<<grid, NarrowTile4::NT, 0, s>>>(p);
  } else if (const int64_t st = (n + SmallTile::BM - 1) / SmallTile::BM *
                                ((d + SmallTile::BN - 1) / SmallTile::BN);
             st <= kCus) {
    const unsigned grid = xcd_grid(st);
    if (dtype == MOE_BF16) down_kernel<uint16_t, SmallTile4, false><<<grid, SmallTile4::NT, 0, s>>>(p);
    else down_kernel<float, SmallTile4, false><<<grid, SmallTile4::NT, 0, s>>>(p);
  } else {
    const unsigned grid = xcd_grid((n + SmallTile::BM - 1) / SmallTile::BM *
                                   ((d + SmallTile::BN - 1) / SmallTile::BN));
    if (dtype == MOE_BF16) down_kernel<uint16_t, SmallTile, false><<<grid, SmallTile::NT, 0, s>>>(p);
    else down_kernel<float, SmallTile, false><<<grid, SmallTile::NT, 0, s>>>(p);
  }
}

hipError_t launch_down_combine(int dtype, const void* h, int64_t n, int d, int Is,
                               const void* w_down, const float* y, const float* weights,
                               int64_t t0, int k, void* out, hipStream_t s) {
  if (n <= 0 || Is <= 0) return hipSuccess;
  ProfScope prof(MOE_STAGE_DOWN_SHARED_COMBINE, s);
  DownParams p{};
  p.h = h; p.n = n; p.d = d; p.K = Is; p.w = w_down; p.line_down_off = 0;
  p.row_slot = nullptr; p.out = nullptr; p.clk = prof_clock(MOE_STAGE_DOWN_SHARED_COMBINE);
  p.y = y; p.wts = weights; p.t0 = t0; p.k = k; p.cout = out;
  down_dense(dtype, p, n, d, s);
  return hipGetLastError();
}

}  // namespace moe
