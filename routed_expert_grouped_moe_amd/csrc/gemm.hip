// GEMMs of the layer on CDNA4 matrix cores: the router, each expert's gate/up projection with
// the fused silu(gate)*up epilogue, and each expert's down projection.
//
// Every GEMM here is X W^T with both operands K-contiguous (x rows and weight rows), tiled
// 128 x 128 per workgroup, K staged through LDS 128 bytes per row at a time (double buffered,
// one barrier per stage). The four waves of a workgroup each own a 64 x 64 block built from
// 4 x 4 MFMA blocks of 16 x 16: v_mfma_f32_16x16x32_bf16 for bf16 storage and
// v_mfma_f32_16x16x4_f32 for fp32 storage, fp32 accumulation in both.
//
// Row invariance (what makes chunked prefill equal the batched pass bit for bit): every
// output element is one token row against one weight row, accumulated over K in the same
// stage order with the same instruction, whatever tile, group size or chunk the row falls
// in. No split-K, no shape-dependent kernel choice, no atomics. This is the property the
// exact deep prefill page ("Flash Next EXL3: exact deep prefill", opening section) asks of
// its GU/down kernels: the same bytes at every chunk size.
#include "device_common.h"
#include "moe_internal.h"
#include "profile.h"

namespace moe {
namespace {

constexpr int kRowBytes = 128;                          // K bytes per row per stage
constexpr int kLdsPitch = kRowBytes + 16;               // padded LDS row pitch
constexpr int kStageBytes = (kBM + kBN) * kLdsPitch;    // A tile + B tile of one stage
constexpr int kLdsBytes = 2 * kStageBytes;              // double buffer: 73,728 bytes

template <typename T> struct Mma;

// bf16: one stage = 64 K elements = 2 MFMA steps of 32. Lane l supplies row (l & 15) and the
// 8 consecutive K elements starting at 8 * (l >> 4) of the step, for A and B alike.
template <> struct Mma<uint16_t> {
  static constexpr int kStageElems = kRowBytes / 2;
  static __device__ __forceinline__ void stage(const char* la, const char* lb,
                                               const int (&arow)[4], const int (&brow)[4],
                                               int kq, f32x4_t (&acc)[4][4]) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8_t a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = *reinterpret_cast<const bf16x8_t*>(la + arow[i] * kLdsPitch + ks * 64 + kq * 16);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[j] = *reinterpret_cast<const bf16x8_t*>(lb + brow[j] * kLdsPitch + ks * 64 + kq * 16);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }
};

// fp32: one stage = 32 K elements = 8 MFMA steps of 4; lane l supplies element (l >> 4).
template <> struct Mma<float> {
  static constexpr int kStageElems = kRowBytes / 4;
  static __device__ __forceinline__ void stage(const char* la, const char* lb,
                                               const int (&arow)[4], const int (&brow)[4],
                                               int kq, f32x4_t (&acc)[4][4]) {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = *reinterpret_cast<const float*>(la + arow[i] * kLdsPitch + (ks * 4 + kq) * 4);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[j] = *reinterpret_cast<const float*>(lb + brow[j] * kLdsPitch + (ks * 4 + kq) * 4);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }
};

// Tile mainloop. Thread t stages rows (t >> 3) + 32 q (q = 0..3) of the A and B tiles, 16 bytes
// at byte (t & 7) * 16 of each 128-byte stage; pa[q] / pb[q] point at those rows' first byte.
// Rows past the end of A or B point at a valid row instead: an MFMA output element depends
// only on its own A row and B column, so those rows and columns are computed and dropped.
// kPairedGU: the B tile holds 64 gate rows then 64 matching up rows, and wave column wn takes
// gate rows wn*32.. and up rows 64 + wn*32.., so that each lane holds gate and up of the same
// output column (acc[i][j] and acc[i][j + 2], j = 0, 1).
template <typename T, bool kPairedGU>
__device__ __forceinline__ void mainloop(const char* const (&pa)[4], const char* const (&pb)[4],
                                         int nk, char* lds, f32x4_t (&acc)[4][4]) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, kq = lane >> 4, l16 = lane & 15;
  const int seg = tid & 7, srow = tid >> 3;
  int arow[4], brow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) arow[i] = wm * 64 + i * 16 + l16;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int b = kPairedGU ? ((j < 2) ? wn * 32 + j * 16 : 64 + wn * 32 + (j - 2) * 16)
                            : wn * 64 + j * 16;
    brow[j] = b + l16;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  uint4 ra0, ra1, ra2, ra3, rb0, rb1, rb2, rb3;
  const int st_off = srow * kLdsPitch + seg * 16;
#define MOE_GLOAD(kb)                                                                     \
  do {                                                                                    \
    const int off_ = (kb) * kRowBytes + seg * 16;                                         \
    ra0 = *reinterpret_cast<const uint4*>(pa[0] + off_);                              \
    ra1 = *reinterpret_cast<const uint4*>(pa[1] + off_);                              \
    ra2 = *reinterpret_cast<const uint4*>(pa[2] + off_);                              \
    ra3 = *reinterpret_cast<const uint4*>(pa[3] + off_);                              \
    rb0 = *reinterpret_cast<const uint4*>(pb[0] + off_);                              \
    rb1 = *reinterpret_cast<const uint4*>(pb[1] + off_);                              \
    rb2 = *reinterpret_cast<const uint4*>(pb[2] + off_);                              \
    rb3 = *reinterpret_cast<const uint4*>(pb[3] + off_);                              \
  } while (0)
#define MOE_SSTORE(buf)                                                                   \
  do {                                                                                    \
    char* b_ = (buf) + st_off;                                                            \
    *reinterpret_cast<uint4*>(b_ + 0 * 32 * kLdsPitch) = ra0;                             \
    *reinterpret_cast<uint4*>(b_ + 1 * 32 * kLdsPitch) = ra1;                             \
    *reinterpret_cast<uint4*>(b_ + 2 * 32 * kLdsPitch) = ra2;                             \
    *reinterpret_cast<uint4*>(b_ + 3 * 32 * kLdsPitch) = ra3;                             \
    *reinterpret_cast<uint4*>(b_ + (kBM + 0 * 32) * kLdsPitch) = rb0;                     \
    *reinterpret_cast<uint4*>(b_ + (kBM + 1 * 32) * kLdsPitch) = rb1;                     \
    *reinterpret_cast<uint4*>(b_ + (kBM + 2 * 32) * kLdsPitch) = rb2;                     \
    *reinterpret_cast<uint4*>(b_ + (kBM + 3 * 32) * kLdsPitch) = rb3;                     \
  } while (0)

  MOE_GLOAD(0);
  MOE_SSTORE(lds);
  __syncthreads();
  for (int kb = 0; kb < nk; ++kb) {
    const char* cur = lds + (kb & 1) * kStageBytes;
    const bool more = kb + 1 < nk;
    if (more) MOE_GLOAD(kb + 1);
    Mma<T>::stage(cur, cur + kBM * kLdsPitch, arow, brow, kq, acc);
    if (more) MOE_SSTORE(lds + ((kb + 1) & 1) * kStageBytes);
    __syncthreads();
  }
#undef MOE_GLOAD
#undef MOE_SSTORE
}

// Output coordinates of accumulator element acc[i][j][r] of this lane (non-paired layout):
//   tile row = wm*64 + i*16 + 4*(lane >> 4) + r, tile column = wn*64 + j*16 + (lane & 15).

struct GuParams {
  const void* x;          // [T, d] prompt rows
  int64_t t0;             // first prompt row of the chunk
  int64_t n;              // dense: rows of the chunk
  int d, I;               // K and h width
  const void* w;          // dense: [2I, d] gate/up weights
  GemmGroups g;           // grouped: routed experts
  const int32_t* row_tok; // grouped: chunk-local token of each permuted row
  void* h;                // [rows, I] out
  bool grouped;
};

template <typename T>
__global__ __launch_bounds__(kThreads) void gu_kernel(GuParams p) {
  __shared__ __align__(16) char lds[kLdsBytes];
  const int tid = threadIdx.x;
  const int n0h = blockIdx.x * kGuHCols;
  int64_t row0;
  int rows;
  const char* wbase;
  if (p.grouped) {
    const int ti = p.g.tile_lo + static_cast<int>(blockIdx.y);
    if (ti >= *p.g.n_mtiles) return;
    const MTile mt = p.g.mtiles[ti];
    row0 = static_cast<int64_t>(p.g.offsets[mt.group]) + mt.m0;
    rows = min(kBM, p.g.counts[mt.group] - mt.m0);
    wbase = static_cast<const char*>(p.g.wtab[mt.group]);
  } else {
    row0 = static_cast<int64_t>(blockIdx.y) * kBM;
    rows = static_cast<int>(min<int64_t>(kBM, p.n - row0));
    wbase = static_cast<const char*>(p.w);
  }
  const bool missing = wbase == nullptr;   // offloaded expert that was not staged
  const size_t rowb = static_cast<size_t>(p.d) * sizeof(T);
  const char* pa[4];
  const char* pb[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int trow = (tid >> 3) + 32 * q;
    const int arow = trow < rows ? trow : 0;
    const int64_t tok = p.grouped ? p.row_tok[row0 + arow] : row0 + arow;
    pa[q] = static_cast<const char*>(p.x) + (p.t0 + tok) * rowb;
    const int64_t wrow = (trow < 64) ? n0h + trow : p.I + n0h + (trow - 64);
    pb[q] = wbase + wrow * rowb;
  }
  f32x4_t acc[4][4];
  if (!missing) mainloop<T, true>(pa, pb, p.d / Mma<T>::kStageElems, lds, acc);

  const int lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
  T* h = static_cast<T*>(p.h);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int trow = wm * 64 + i * 16 + 4 * (lane >> 4) + r;
      if (trow >= rows) continue;
      T* hrow = h + (row0 + trow) * static_cast<int64_t>(p.I);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = n0h + wn * 32 + j * 16 + (lane & 15);
        const float hv = missing ? __builtin_nanf("") : silu_f32(acc[i][j][r]) * acc[i][j + 2][r];
        hrow[col] = Elt<T>::store(hv);
      }
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
  float* out;             // grouped: Y [n*k, d]; dense: S [n, d]
  bool grouped;
};

template <typename T>
__global__ __launch_bounds__(kThreads) void down_kernel(DownParams p) {
  __shared__ __align__(16) char lds[kLdsBytes];
  const int tid = threadIdx.x;
  const int n0 = blockIdx.x * kBN;
  int64_t row0;
  int rows;
  const char* wbase;
  if (p.grouped) {
    const int ti = p.g.tile_lo + static_cast<int>(blockIdx.y);
    if (ti >= *p.g.n_mtiles) return;
    const MTile mt = p.g.mtiles[ti];
    row0 = static_cast<int64_t>(p.g.offsets[mt.group]) + mt.m0;
    rows = min(kBM, p.g.counts[mt.group] - mt.m0);
    const char* line = static_cast<const char*>(p.g.wtab[mt.group]);
    wbase = line ? line + p.line_down_off * static_cast<int64_t>(sizeof(T)) : nullptr;
  } else {
    row0 = static_cast<int64_t>(blockIdx.y) * kBM;
    rows = static_cast<int>(min<int64_t>(kBM, p.n - row0));
    wbase = static_cast<const char*>(p.w);
  }
  const bool missing = wbase == nullptr;
  const size_t rowb = static_cast<size_t>(p.K) * sizeof(T);
  const char* pa[4];
  const char* pb[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int trow = (tid >> 3) + 32 * q;
    pa[q] = static_cast<const char*>(p.h) + (row0 + (trow < rows ? trow : 0)) * rowb;
    pb[q] = wbase + static_cast<int64_t>(n0 + trow < p.d ? n0 + trow : n0) * rowb;
  }
  f32x4_t acc[4][4];
  if (!missing) mainloop<T, false>(pa, pb, p.K / Mma<T>::kStageElems, lds, acc);

  const int lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int trow = wm * 64 + i * 16 + 4 * (lane >> 4) + r;
      if (trow >= rows) continue;
      const int64_t orow = p.grouped ? p.row_slot[row0 + trow] : row0 + trow;
      float* o = p.out + orow * static_cast<int64_t>(p.d);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = n0 + wn * 64 + j * 16 + (lane & 15);
        if (col < p.d) o[col] = missing ? __builtin_nanf("") : acc[i][j][r];
      }
    }
}

struct RouterParams {
  const void* x;
  const void* w;
  const float* bias;
  float* logits;
  int64_t T;
  int d, E;
};

template <typename T>
__global__ __launch_bounds__(kThreads) void router_kernel(RouterParams p) {
  __shared__ __align__(16) char lds[kLdsBytes];
  const int tid = threadIdx.x;
  const int n0 = blockIdx.x * kBN;
  const int64_t row0 = static_cast<int64_t>(blockIdx.y) * kBM;
  const int rows = static_cast<int>(min<int64_t>(kBM, p.T - row0));
  const size_t rowb = static_cast<size_t>(p.d) * sizeof(T);
  const char* pa[4];
  const char* pb[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int trow = (tid >> 3) + 32 * q;
    pa[q] = static_cast<const char*>(p.x) + (row0 + (trow < rows ? trow : 0)) * rowb;
    pb[q] = static_cast<const char*>(p.w) +
            static_cast<int64_t>(n0 + trow < p.E ? n0 + trow : n0) * rowb;
  }
  f32x4_t acc[4][4];
  mainloop<T, false>(pa, pb, p.d / Mma<T>::kStageElems, lds, acc);

  const int lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int trow = wm * 64 + i * 16 + 4 * (lane >> 4) + r;
      if (trow >= rows) continue;
      float* o = p.logits + (row0 + trow) * static_cast<int64_t>(p.E);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = n0 + wn * 64 + j * 16 + (lane & 15);
        if (col < p.E) o[col] = acc[i][j][r] + (p.bias ? p.bias[col] : 0.0f);
      }
    }
}

}  // namespace

hipError_t launch_router_gemm(int dtype, const void* x, const void* w_router, const float* bias,
                              int64_t T, int d, int E, float* logits, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  ProfScope prof(MOE_STAGE_ROUTER, s);
  RouterParams p{x, w_router, bias, logits, T, d, E};
  dim3 grid((E + kBN - 1) / kBN, static_cast<unsigned>((T + kBM - 1) / kBM));
  if (dtype == MOE_BF16) router_kernel<uint16_t><<<grid, kThreads, 0, s>>>(p);
  else router_kernel<float><<<grid, kThreads, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_gu_routed(int dtype, const void* x, int64_t t0, int d, int I,
                            const GemmGroups& g, const int32_t* row_tok, void* h, hipStream_t s) {
  if (g.tile_cap <= 0) return hipSuccess;
  ProfScope prof(MOE_STAGE_GU_ROUTED, s);
  GuParams p{};
  p.x = x; p.t0 = t0; p.n = 0; p.d = d; p.I = I; p.w = nullptr; p.g = g;
  p.row_tok = row_tok; p.h = h; p.grouped = true;
  dim3 grid(I / kGuHCols, g.tile_cap);
  if (dtype == MOE_BF16) gu_kernel<uint16_t><<<grid, kThreads, 0, s>>>(p);
  else gu_kernel<float><<<grid, kThreads, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_gu_dense(int dtype, const void* x, int64_t t0, int64_t n, int d, int Is,
                           const void* w_gu, void* h, hipStream_t s) {
  if (n <= 0 || Is <= 0) return hipSuccess;
  ProfScope prof(MOE_STAGE_GU_SHARED, s);
  GuParams p{};
  p.x = x; p.t0 = t0; p.n = n; p.d = d; p.I = Is; p.w = w_gu; p.row_tok = nullptr;
  p.h = h; p.grouped = false;
  dim3 grid(Is / kGuHCols, static_cast<unsigned>((n + kBM - 1) / kBM));
  if (dtype == MOE_BF16) gu_kernel<uint16_t><<<grid, kThreads, 0, s>>>(p);
  else gu_kernel<float><<<grid, kThreads, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_down_routed(int dtype, const void* h, int d, int I, const GemmGroups& g,
                              const int32_t* row_slot, float* y, hipStream_t s) {
  if (g.tile_cap <= 0) return hipSuccess;
  ProfScope prof(MOE_STAGE_DOWN_ROUTED, s);
  DownParams p{};
  p.h = h; p.n = 0; p.d = d; p.K = I; p.w = nullptr; p.g = g;
  p.line_down_off = 2LL * I * d; p.row_slot = row_slot; p.out = y; p.grouped = true;
  dim3 grid((d + kBN - 1) / kBN, g.tile_cap);
  if (dtype == MOE_BF16) down_kernel<uint16_t><<<grid, kThreads, 0, s>>>(p);
  else down_kernel<float><<<grid, kThreads, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_down_dense(int dtype, const void* h, int64_t n, int d, int Is,
                             const void* w_down, float* out, hipStream_t s) {
  if (n <= 0 || Is <= 0) return hipSuccess;
  ProfScope prof(MOE_STAGE_DOWN_SHARED, s);
  DownParams p{};
  p.h = h; p.n = n; p.d = d; p.K = Is; p.w = w_down; p.line_down_off = 0;
  p.row_slot = nullptr; p.out = out; p.grouped = false;
  dim3 grid((d + kBN - 1) / kBN, static_cast<unsigned>((n + kBM - 1) / kBM));
  if (dtype == MOE_BF16) down_kernel<uint16_t><<<grid, kThreads, 0, s>>>(p);
  else down_kernel<float><<<grid, kThreads, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace moe
