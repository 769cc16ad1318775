// kd_gemm.hpp -- one NT matrix-core GEMM for gfx950, shared by the four
// contractions of the fused chunked KL loss.
//
// C[m, n] = sum_k A[m, k] * B[n, k], both operands row-major with K
// contiguous ("NT").  Every contraction of the method is brought into this
// form: the logits of a chunk are z^T = W * H_c^T (A = W, B = H_c); the
// hidden gradient is dH = G * W (A = G, B = W^T); the head gradient is
// dW = G^T * H_c (A = G^T, B = H_c^T).  The transposed copies (W^T per call,
// H_c^T per chunk, G^T written by the gradient epilogue) cost a few percent
// of the traffic and let a single LDS layout and MFMA schedule serve all.
//
// Tiling.  A block computes a BM x BN tile with 64 * WM * WN threads; each
// wave owns a (BM/WM) x (BN/WN) sub-tile made of 32x32 MFMA tiles.  K is
// consumed in steps of 128 bytes per row (64 bf16 or 32 fp32).  Tiles are
// staged through LDS, double-buffered, with a 16-byte XOR swizzle (unit u of
// row r is stored at unit u ^ (r & 7)) so that both the 16-byte global->LDS
// writes and the 16-byte fragment reads are bank-conflict free.
//
// Bounds.  Operand rows past the matrix end are read through buffer
// resources whose size ends at the last valid row, so the hardware returns
// zeros for them; the K extent of every operand is padded with zeros to a
// multiple of 128 bytes by the caller.
//
// The MFMA accumulator layout (32x32 tiles): register r of lane l holds
// C[8*(r/4) + 4*(l/32) + r%4][l%32].  So each lane holds one column n and a
// strip of rows m in registers -- with m along the vocabulary, row statistics
// over the vocabulary reduce mostly inside a lane.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Element tags.  Storage of bf16 is uint16_t bit patterns.
struct Bf16 { typedef uint16_t T; static constexpr int kBytes = 2; };
struct F32 { typedef float T; static constexpr int kBytes = 4; };

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t nbytes) {
  // word3 = 0x00020000: raw (untyped) buffer on gfx9-family parts.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nbytes, 0x00020000);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// fp32 -> bf16, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <class E> __device__ __forceinline__ float load_elem(const typename E::T* p);
template <> __device__ __forceinline__ float load_elem<Bf16>(const uint16_t* p) { return bf16_to_f32(*p); }
template <> __device__ __forceinline__ float load_elem<F32>(const float* p) { return *p; }
template <class E> __device__ __forceinline__ typename E::T store_cvt(float f);
template <> __device__ __forceinline__ uint16_t store_cvt<Bf16>(float f) { return f32_to_bf16(f); }
template <> __device__ __forceinline__ float store_cvt<F32>(float f) { return f; }

// One 32-byte K group per lane pair: each half-wave supplies one 16-byte unit
// of K for its row/column.  The K order inside a group is irrelevant to the
// sum as long as A and B use the same order, which they do.
template <class E> __device__ __forceinline__ void mfma_group(f32x16& acc, u32x4 a, u32x4 b);
template <> __device__ __forceinline__ void mfma_group<Bf16>(f32x16& acc, u32x4 a, u32x4 b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}
template <> __device__ __forceinline__ void mfma_group<F32>(f32x16& acc, u32x4 a, u32x4 b) {
  f32x4 fa = __builtin_bit_cast(f32x4, a), fb = __builtin_bit_cast(f32x4, b);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa.x, fb.x, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa.y, fb.y, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa.z, fb.z, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa.w, fb.w, acc, 0, 0, 0);
}

struct GemmShape {
  const void* A;      // [M, lda] elements, K-contiguous
  const void* B;      // [N, ldb]
  int64_t lda, ldb;   // row strides in elements
  int M, N;           // valid rows of A and B
  int k_tiles;        // 128-byte K steps in the whole product
  int k_tiles_per_split;
  int tiles_m, tiles_n, splits;
};

// Position of this block's tile.  Blocks are dispatched round-robin over the
// 8 XCDs; consecutive logical tiles are sent to the same XCD so that the
// blocks sharing an A tile (same m, consecutive n) hit the same L2.
struct TilePos { int tm, tn, split; bool valid; };

__device__ __forceinline__ TilePos tile_position(const GemmShape& g) {
  const int nb = g.tiles_m * g.tiles_n * g.splits;
  const int per = gridDim.x >> 3;              // gridDim.x is a multiple of 8
  const int lin = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
  TilePos p;
  p.valid = lin < nb;
  const int mn = g.tiles_m * g.tiles_n;
  p.split = lin / mn;
  const int r = lin - p.split * mn;
  p.tm = r / g.tiles_n;
  p.tn = r - p.tm * g.tiles_n;
  return p;
}

// Per-wave epilogue context.
struct EpiCtx {
  int m0;     // first row (M) of the wave's sub-tile in C
  int n0;     // first column (N) of the wave's sub-tile in C
  int lane;
  int split;
  int tm, tn;
  int wm, wn;
  char* smem;
};

template <class E, int BM, int BN, int WM, int WN>
struct GemmCfg {
  static constexpr int kThreads = 64 * WM * WN;
  static constexpr int TM = BM / WM, TN = BN / WN;
  static constexpr int FM = TM / 32, FN = TN / 32;
  static constexpr int kLdsStage = (BM + BN) * 128;
  static constexpr int kLds = 2 * kLdsStage;
  static constexpr int UA = BM * 8 / kThreads;   // 16-byte units of A per thread per stage
  static constexpr int UB = BN * 8 / kThreads;
  static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be a multiple of 32");
  static_assert((BM * 8) % kThreads == 0 && (BN * 8) % kThreads == 0, "loader split");
};

template <class E, int BM, int BN, int WM, int WN, class Epi>
__global__ __launch_bounds__(64 * WM * WN) void gemm_nt_kernel(GemmShape g, Epi epi) {
  typedef GemmCfg<E, BM, BN, WM, WN> C;
  __shared__ __attribute__((aligned(16))) char smem[C::kLds];

  const TilePos pos = tile_position(g);
  if (!pos.valid) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int wm = wid / WN, wn = wid - (wid / WN) * WN;

  const int kt0 = pos.split * g.k_tiles_per_split;
  int kt1 = kt0 + g.k_tiles_per_split;
  if (kt1 > g.k_tiles) kt1 = g.k_tiles;
  const int nk = kt1 > kt0 ? kt1 - kt0 : 0;

  const int rowsA = min(BM, g.M - pos.tm * BM);
  const int rowsB = min(BN, g.N - pos.tn * BN);
  const int64_t strideA = g.lda * E::kBytes, strideB = g.ldb * E::kBytes;
  const char* baseA = (const char*)g.A + (int64_t)pos.tm * BM * strideA + (int64_t)kt0 * 128;
  const char* baseB = (const char*)g.B + (int64_t)pos.tn * BN * strideB + (int64_t)kt0 * 128;
  // rowsA may be <= 0 only for an empty matrix, which the host never launches.
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(baseA, (uint32_t)(rowsA * strideA - kt0 * 128));
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(baseB, (uint32_t)(rowsB * strideB - kt0 * 128));

  // Loader: unit q = tid + kThreads * i covers row q >> 3, 16-byte unit q & 7.
  uint32_t goffA[C::UA], goffB[C::UB];
  uint32_t loffA[C::UA], loffB[C::UB];
#pragma unroll
  for (int i = 0; i < C::UA; ++i) {
    const int q = tid + C::kThreads * i, r = q >> 3, u = q & 7;
    goffA[i] = (uint32_t)(r * strideA + u * 16);
    loffA[i] = (uint32_t)(r * 128 + ((u ^ (r & 7)) << 4));
  }
#pragma unroll
  for (int i = 0; i < C::UB; ++i) {
    const int q = tid + C::kThreads * i, r = q >> 3, u = q & 7;
    goffB[i] = (uint32_t)(r * strideB + u * 16);
    loffB[i] = (uint32_t)(BM * 128 + r * 128 + ((u ^ (r & 7)) << 4));
  }

  f32x16 acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  u32x4 sa[C::UA], sb[C::UB];
  auto gload = [&](int kt) {
    const uint32_t ko = (uint32_t)kt * 128u;
#pragma unroll
    for (int i = 0; i < C::UA; ++i) sa[i] = __builtin_amdgcn_raw_buffer_load_b128(ra, goffA[i] + ko, 0, 0);
#pragma unroll
    for (int i = 0; i < C::UB; ++i) sb[i] = __builtin_amdgcn_raw_buffer_load_b128(rb, goffB[i] + ko, 0, 0);
  };
  auto lstore = [&](int stage) {
    char* s = smem + stage * C::kLdsStage;
#pragma unroll
    for (int i = 0; i < C::UA; ++i) *(u32x4*)(s + loffA[i]) = sa[i];
#pragma unroll
    for (int i = 0; i < C::UB; ++i) *(u32x4*)(s + loffB[i]) = sb[i];
  };

  // Fragment read offsets: row (lane & 31) of each 32-row MFMA tile, unit
  // 2*grp + (lane >> 5), swizzled by (row & 7) == (lane & 7).
  const int frow = lane & 31, fhalf = lane >> 5, fsw = lane & 7;
  const uint32_t aRow0 = (uint32_t)((wm * C::TM + frow) * 128);
  const uint32_t bRow0 = (uint32_t)(BM * 128 + (wn * C::TN + frow) * 128);

  if (nk > 0) {
    gload(0);
    lstore(0);
    __syncthreads();
  }
  for (int it = 0; it < nk; ++it) {
    const int cur = it & 1;
    if (it + 1 < nk) gload(it + 1);
    const char* s = smem + cur * C::kLdsStage;
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
      const uint32_t uoff = (uint32_t)((((2 * grp + fhalf) ^ fsw)) << 4);
      u32x4 fa[C::FM], fb[C::FN];
#pragma unroll
      for (int i = 0; i < C::FM; ++i) fa[i] = *(const u32x4*)(s + aRow0 + i * 32 * 128 + uoff);
#pragma unroll
      for (int j = 0; j < C::FN; ++j) fb[j] = *(const u32x4*)(s + bRow0 + j * 32 * 128 + uoff);
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j) mfma_group<E>(acc[i][j], fa[i], fb[j]);
    }
    if (it + 1 < nk) lstore(cur ^ 1);
    __syncthreads();
  }

  EpiCtx ctx;
  ctx.m0 = pos.tm * BM + wm * C::TM;
  ctx.n0 = pos.tn * BN + wn * C::TN;
  ctx.lane = lane;
  ctx.split = pos.split;
  ctx.tm = pos.tm;
  ctx.tn = pos.tn;
  ctx.wm = wm;
  ctx.wn = wn;
  ctx.smem = smem;
  epi.template apply<C::FM, C::FN>(acc, ctx);
}

// Row (M) index of register r of lane l inside a 32x32 tile, column index.
__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }
__device__ __forceinline__ int acc_col(int lane) { return lane & 31; }

}  // namespace kd
