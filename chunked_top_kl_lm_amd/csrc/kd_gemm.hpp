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
// wave owns a (BM/WM) x (BN/WN) sub-tile made of 32x32x16 (bf16) or 32x32x2
// (fp32) MFMA tiles.  K is consumed in stages of 64 bytes per row (32 bf16 or
// 16 fp32), moved global -> LDS by direct LDS-DMA loads into a ring of STAGES
// buffers (see gemm_nt_kernel).
//
// Bounds.  Operand rows past the matrix end are read through buffer
// resources whose size ends at the last valid row, so the hardware returns
// zeros for them; the K extent of every operand is padded with zeros to a
// multiple of 64 bytes by the caller.
//
// The MFMA accumulator layout (32x32 tiles): register r of lane l holds
// C[8*(r/4) + 4*(l/32) + r%4][l%32].  So each lane holds one column n and a
// strip of rows m in registers -- with m along the vocabulary, row statistics
// over the vocabulary reduce mostly inside a lane.
#pragma once

#include <hip/hip_runtime.h>
#include <type_traits>
#include <stdint.h>

#include "kd_layout.hpp"

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

// fp32 -> bf16, round to nearest even, NaN kept NaN (quiet bit set, payload
// truncated).  gfx950 has this as v_cvt_pk_bf16_f32, two values per
// instruction; over all 2^32 fp32 bit patterns its results equal the integer
// form ((u + 0x7fff + bit 16 of u) >> 16, NaN: (u >> 16) | 0x40) bit for bit.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
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
  int group_m;        // tile order: groups of group_m row tiles x all column tiles
};

// Position of this block's tile.  Linear tile order: split-K slice, then
// groups of group_m row tiles x all column tiles, row index fastest inside a
// group, so that a window of consecutive tiles shares both its A and B
// tiles.  Blocks are dispatched round-robin over the 8 XCDs; each XCD is
// given one contiguous range of that order, so the blocks an XCD runs at
// the same time share their operands in its L2.
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
  const int span = g.group_m * g.tiles_n;      // tiles per full group
  const int grp = r / span;
  const int w = r - grp * span;
  const int gm = min(g.group_m, g.tiles_m - grp * g.group_m);
  p.tm = grp * g.group_m + w % gm;
  p.tn = w / gm;
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
  int wid, nwaves;
  char* smem;       // the LDS ring (free once the main loop has ended)
  int smem_bytes;   // its size
  uint32_t pf[12];  // values an epilogue loaded ahead (see prefetch below)
};

// Epilogue prefetch.  An epilogue that reads small per-tile inputs (hit
// lists, row scales) may declare kPrefetchSteps = n > 0 and a method
// prefetch<FM, FN>(EpiCtx&, int step): the kernel calls it with step 0 before
// the first K stage and with steps 1..n after main-loop stages 0, S-1, ...,
// (n-1)(S-1) (S = STAGES), so each step's loads have returned before the next
// step (the wait of a stage leaves only the DMA of the S-2 newer stages in
// flight), and the latency of dependent loads hides behind the MFMAs instead
// of stalling the epilogue.
template <class T, class = void>
struct PrefetchSteps {
  static constexpr int value = 0;
};
template <class T>
struct PrefetchSteps<T, std::void_t<decltype(T::kPrefetchSteps)>> {
  static constexpr int value = T::kPrefetchSteps;
};

// ---------------------------------------------------------------------------
// LDS staging.  Each stage holds A [BM rows x 64 B] then B [BN rows x 64 B].  A wave's
// LDS-DMA instruction writes 1 KB of consecutive LDS (lane l -> bytes
// 16l..16l+15), i.e. 16 rows of 64 B; the swizzle is applied on the global
// side: the lane that fills slot s of row r fetches logical 16-byte unit
// s ^ f(r), f(r) = (r >> 2) & 3.  gfx950 serves a 128-bit LDS read in 4
// cycles when conflict-free (256 B/clk); with this f the MFMA fragment reads
// (32 consecutive rows, two units per row) measure conflict-free with the
// SQ_LDS_BANK_CONFLICT counter, whereas f = ((r>>1)^(r>>3)) & 3 and the
// 128-byte-row layout with f = r & 7 measure 2-way conflicts.
//
// Ordering: the loads for stage `it` are waited for with s_waitcnt vmcnt
// (counting only this wave's later-issued loads), then a workgroup barrier
// makes every wave's LDS writes visible; the stage overwritten next is the
// one all waves finished reading before that same barrier.
// ---------------------------------------------------------------------------
// (swz<RB> in kd_layout.hpp is the 16-byte slot permutation of an LDS row
// of RB bytes; dma_src_offset the source offset it implies.)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <class E, int BM, int BN, int WM, int WN, int STAGES, int RB_ = 64>
struct PipeCfg {
  static constexpr int kThreads = 64 * WM * WN;
  static constexpr int NW = WM * WN;
  static constexpr int TM = BM / WM, TN = BN / WN;
  static constexpr int FM = TM / 32, FN = TN / 32;
  static constexpr int RB = RB_;                // bytes of K per row per stage
  static constexpr int GROUPS = RB / 32;        // 32-byte K groups per stage
  static constexpr int RPD = 1024 / RB;         // rows per 1 KB DMA instruction
  static constexpr int kStage = (BM + BN) * RB;
  static constexpr int kLds = STAGES * kStage;
  static constexpr int IA = BM / RPD / NW;      // DMA instructions per wave per stage (A)
  static constexpr int IB = BN / RPD / NW;
  static constexpr int kPer = IA + IB;
  static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be a multiple of 32");
  static_assert((BM / RPD) % NW == 0 && (BN / RPD) % NW == 0, "DMA split");
  static_assert(STAGES >= 2 && (STAGES - 1) * (IA + IB) < 64, "vmcnt range");
  static_assert(GROUPS % 2 == 0, "fragment ping-pong needs an even group count");
};

template <class C, int BM>
__device__ __forceinline__ void dma_stage(char* s, __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb,
                                          const uint32_t* voffA, const uint32_t* voffB, int wid, uint32_t ko) {
#pragma unroll
  for (int i = 0; i < C::IA; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (__attribute__((address_space(3))) void*)(s + (wid + C::NW * i) * 1024),
                                             16, voffA[i] + ko, 0, 0, 0);
#pragma unroll
  for (int i = 0; i < C::IB; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rb, (__attribute__((address_space(3))) void*)(s + BM * C::RB + (wid + C::NW * i) * 1024), 16, voffB[i] + ko, 0,
        0, 0);
}

// ---------------------------------------------------------------------------
// Main loop.  The per-stage barrier sits in the middle of a stage, so that
// the MFMA pipe never drains on it:
//
//   iteration it (fa0/fb0 already hold K-group 0 of stage it; a K-group is
//   32 bytes of K, one 16-byte unit per half-wave):
//     read K-group 1 fragments of stage it        } interleaved with the
//     MFMAs of K-group 0                          } MFMAs
//     wait for this wave's ds_reads and for stage it+1's DMA; barrier
//     DMA of stage it+STAGES into the buffer of stage it (all waves are
//     done reading it), read K-group 0 of stage it+1, MFMAs of K-group 1
//
// The DMA and ds_read issues are spread between MFMAs with
// sched_group_barrier so the two waves of a SIMD keep its MFMA pipe fed.
// ---------------------------------------------------------------------------
template <class C>
__device__ __forceinline__ void read_frags(const char* s, uint32_t aRow0, uint32_t bRow0, uint32_t uoff,
                                           u32x4 (&fa)[C::FM], u32x4 (&fb)[C::FN]) {
#pragma unroll
  for (int i = 0; i < C::FM; ++i) fa[i] = *(const u32x4*)(s + aRow0 + i * 32 * C::RB + uoff);
#pragma unroll
  for (int j = 0; j < C::FN; ++j) fb[j] = *(const u32x4*)(s + bRow0 + j * 32 * C::RB + uoff);
}

template <class E, class C>
__device__ __forceinline__ void mfma_all(f32x16 (&acc)[C::FM][C::FN], const u32x4 (&fa)[C::FM],
                                         const u32x4 (&fb)[C::FN]) {
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) mfma_group<E>(acc[i][j], fa[i], fb[j]);
}

// Interleave hints for one K-group: MFMAs alternate with `reads` DS reads
// and, for the group that carries the stage refill, with the DMA issues.
template <class C, int ID, bool DMA>
__device__ __forceinline__ void sched_group_hints() {
  if constexpr (DMA) {
#pragma unroll
    for (int z = 0; z < C::kPer; ++z) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, ID);  // 1 MFMA
      __builtin_amdgcn_sched_group_barrier(0x020, 1, ID);  // 1 VMEM (DMA)
    }
  }
#pragma unroll
  for (int z = 0; z < C::FM + C::FN; ++z) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, ID);    // 1 MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, ID);    // 1 DS read
  }
}

// One K stage of the main loop (see gemm_nt_kernel).  MORE: another stage
// follows, so this one ends with the wait / barrier / refill / prefetch.
template <class E, class C, int BM, int STAGES, bool MORE>
__device__ __forceinline__ void gemm_stage(f32x16 (&acc)[C::FM][C::FN], u32x4 (&fa)[2][C::FM], u32x4 (&fb)[2][C::FN],
                                           char* smem, int it, uint32_t aRow0, uint32_t bRow0,
                                           const uint32_t (&uoff)[C::GROUPS], __amdgpu_buffer_rsrc_t ra,
                                           __amdgpu_buffer_rsrc_t rb, const uint32_t* voffA, const uint32_t* voffB,
                                           int wid, uint32_t refill_ko) {
  const char* s = smem + (it % STAGES) * C::kStage;
#pragma unroll
  for (int q = 0; q < C::GROUPS; ++q) {
    const int cur = q & 1, nxt = cur ^ 1;
    if (q + 1 < C::GROUPS) {
      read_frags<C>(s, aRow0, bRow0, uoff[q + 1], fa[nxt], fb[nxt]);
    } else if constexpr (MORE) {
      // this wave's reads of stage `it` have returned; stage it+1 has landed
      __builtin_amdgcn_s_waitcnt(0xC07F);                  // lgkmcnt(0)
      wait_vmcnt<(STAGES - 2) * C::kPer>();
      lds_barrier();
      dma_stage<C, BM>(smem + (it % STAGES) * C::kStage, ra, rb, voffA, voffB, wid, refill_ko);
      read_frags<C>(smem + ((it + 1) % STAGES) * C::kStage, aRow0, bRow0, uoff[0], fa[nxt], fb[nxt]);
    }
    mfma_all<E, C>(acc, fa[cur], fb[cur]);
    if (q + 1 == C::GROUPS) sched_group_hints<C, 2 * C::GROUPS, MORE>();
    else sched_group_hints<C, 2 * C::GROUPS, false>();
  }
}

// One block per output tile (grid = all tiles, rounded up to a multiple of
// 8): the dispatcher hands a CU its next tile as soon as the previous one
// ends.  The 2-stage rings of the tiles in use (112-144 KB of LDS) fit one
// block per CU.
//
// Each stage holds RB bytes of K (GROUPS = RB/32 K-groups).  Fragments are
// read one group ahead into a second register set; before the last group's
// MFMAs the wave waits for its own reads and for the next stage's DMA,
// passes the barrier, refills the buffer it has just consumed, and reads
// group 0 of the next stage.
template <class E, int BM, int BN, int WM, int WN, int STAGES, class Epi, int RB = 64>
__global__ __launch_bounds__(64 * WM * WN) void gemm_nt_kernel(GemmShape g, Epi epi) {
  typedef PipeCfg<E, BM, BN, WM, WN, STAGES, RB> C;
  __shared__ __attribute__((aligned(1024))) char smem[C::kLds];

  const TilePos pos = tile_position(g);
  if (!pos.valid) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int wm = wid / WN, wn = wid - (wid / WN) * WN;

  constexpr int PS = PrefetchSteps<Epi>::value;
  // a prefetch issued after stage `it` has returned by the wait of stage
  // it + STAGES - 1 (that wait leaves only the newer stages' DMA in flight)
  constexpr int PGAP = STAGES - 1;
  EpiCtx ctx;
  ctx.m0 = pos.tm * BM + wm * C::TM;
  ctx.n0 = pos.tn * BN + wn * C::TN;
  ctx.lane = lane;
  ctx.split = pos.split;
  ctx.tm = pos.tm;
  ctx.tn = pos.tn;
  ctx.wm = wm;
  ctx.wn = wn;
  ctx.wid = wid;
  ctx.nwaves = C::NW;
  ctx.smem = smem;
  ctx.smem_bytes = C::kLds;
  if constexpr (PS > 0) epi.template prefetch<C::FM, C::FN>(ctx, 0);

  // g.k_tiles counts RB-byte K stages
  const int kt0 = pos.split * g.k_tiles_per_split;
  int kt1 = kt0 + g.k_tiles_per_split;
  if (kt1 > g.k_tiles) kt1 = g.k_tiles;
  const int nk = kt1 > kt0 ? kt1 - kt0 : 0;

  const int rowsA = min(BM, g.M - pos.tm * BM);
  const int rowsB = min(BN, g.N - pos.tn * BN);
  const int64_t strideA = g.lda * E::kBytes, strideB = g.ldb * E::kBytes;
  const char* baseA = (const char*)g.A + (int64_t)pos.tm * BM * strideA + (int64_t)kt0 * RB;
  const char* baseB = (const char*)g.B + (int64_t)pos.tn * BN * strideB + (int64_t)kt0 * RB;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(baseA, (uint32_t)(rowsA * strideA - kt0 * RB));
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(baseB, (uint32_t)(rowsB * strideB - kt0 * RB));

  // DMA source offsets: lane fills slot (lane % UPR) of row r = RPD*j +
  // lane / UPR of the stage (j = wid + NW*i); that slot holds logical unit
  // slot ^ f(r).
  constexpr int UPR = RB / 16;                             // 16-byte units per row
  uint32_t voffA[C::IA], voffB[C::IB];
#pragma unroll
  for (int i = 0; i < C::IA; ++i) {
    voffA[i] = dma_src_offset<RB>(C::RPD * (wid + C::NW * i) + lane / UPR, lane, strideA);
  }
#pragma unroll
  for (int i = 0; i < C::IB; ++i) {
    voffB[i] = dma_src_offset<RB>(C::RPD * (wid + C::NW * i) + lane / UPR, lane, strideB);
  }

  f32x16 acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // fragment reads: row (lane & 31) of a 32-row MFMA tile, logical unit
  // 2*group + (lane >> 5), at slot unit ^ f(row); f is the same for every
  // 32-row tile of the wave
  const int frow = lane & 31, fhalf = lane >> 5;
  const int fsw = swz<RB>(wm * C::TM + frow);
  const uint32_t aRow0 = (uint32_t)((wm * C::TM + frow) * RB);
  const uint32_t bRow0 = (uint32_t)(BM * RB + (wn * C::TN + frow) * RB);
  uint32_t uoff[C::GROUPS];
#pragma unroll
  for (int q = 0; q < C::GROUPS; ++q) uoff[q] = (uint32_t)(((2 * q + fhalf) ^ fsw) << 4);

  // Stages past the end of K are still issued, at an offset beyond the
  // buffer range: the hardware returns zeros without a memory access.  Every
  // iteration thus issues exactly one stage and the vmcnt bookkeeping is the
  // same constant in all of them.
  auto kofs = [&](int kt) -> uint32_t { return kt < nk ? (uint32_t)kt * RB : 0x80000000u; };

  u32x4 fa[2][C::FM], fb[2][C::FN];
  if (nk > 0) {
#pragma unroll
    for (int st = 0; st < STAGES; ++st) dma_stage<C, BM>(smem + st * C::kStage, ra, rb, voffA, voffB, wid, kofs(st));
    wait_vmcnt<(STAGES - 1) * C::kPer>();                  // stage 0 has landed
    lds_barrier();
    read_frags<C>(smem, aRow0, bRow0, uoff[0], fa[0], fb[0]);

    for (int it = 0; it < nk - 1; ++it) {
      gemm_stage<E, C, BM, STAGES, true>(acc, fa, fb, smem, it, aRow0, bRow0, uoff, ra, rb, voffA, voffB, wid,
                                         kofs(it + STAGES));
      if constexpr (PS > 0)
        if (it % PGAP == 0 && it / PGAP < PS) epi.template prefetch<C::FM, C::FN>(ctx, it / PGAP + 1);
    }
    gemm_stage<E, C, BM, STAGES, false>(acc, fa, fb, smem, nk - 1, aRow0, bRow0, uoff, ra, rb, voffA, voffB, wid, 0u);
    wait_vmcnt<0>();                                       // drain the tail loads before LDS is reused
  }
  if constexpr (PS > 0) {
    // steps a short K loop did not reach, each after the previous one's loads
    for (int s = (nk > 1 ? min((nk - 2) / PGAP + 1, PS) : 0) + 1; s <= PS; ++s) {
      __builtin_amdgcn_s_waitcnt(0);
      epi.template prefetch<C::FM, C::FN>(ctx, s);
    }
    __builtin_amdgcn_s_waitcnt(0);
  }
  lds_barrier();

  epi.template apply<C::FM, C::FN>(acc, ctx);
}

}  // namespace kd
