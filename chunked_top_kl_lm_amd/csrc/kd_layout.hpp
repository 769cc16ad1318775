// kd_layout.hpp -- layout constants and the index arithmetic of the kernels:
// the MFMA accumulator layout, the LDS swizzles, the hit-list entry code and
// the addresses the GEMM epilogues form.  The kernels compute every such
// address through these functions, and tests/index_check.cpp compiles the
// same functions for the host and checks, over swept shapes, that every
// access stays inside its buffer and reaches the element it should.
//
// KD_HD marks them callable from both sides under hipcc; a plain C++
// compiler (the host checks) sees ordinary inline functions.
#pragma once

#include <stddef.h>
#include <stdint.h>

#ifdef __HIPCC__
#define KD_HD __host__ __device__
#else
#define KD_HD
#endif

namespace kd {

constexpr int kMaxK = 4096;        // largest cache width K
constexpr int kHitV = 128;         // vocabulary rows of one forward-GEMM wave tile
constexpr int kHitT = 64;          // chunk rows of one forward-GEMM wave tile
constexpr int kMergeStrips = 64;   // strips merged per first-level logsumexp group
constexpr int kBlockRows = 32;     // cache builder: vocabulary rows per block maximum
constexpr int kFbBatch = 1024;     // cache builder: ids per batch of the exact fallback

KD_HD constexpr int imin(int a, int b) { return a < b ? a : b; }
KD_HD constexpr int imax(int a, int b) { return a > b ? a : b; }

// ---------------------------------------------------------------------------
// MFMA 32x32 accumulator layout (v_mfma_f32_32x32x16_bf16 / 32x32x2_f32):
// register r of lane l holds C[acc_row(r, l)][acc_col(l)].
// ---------------------------------------------------------------------------
KD_HD constexpr int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }
KD_HD constexpr int acc_col(int lane) { return lane & 31; }
// The inverse: the register and the lane that hold row rr (0..31) and column
// col of a 32x32 tile.
KD_HD constexpr int acc_reg_of(int rr) { return 4 * (rr >> 3) + (rr & 3); }
KD_HD constexpr int acc_lane_of(int rr, int col) { return (col & 31) + 32 * ((rr >> 2) & 1); }

// ---------------------------------------------------------------------------
// GEMM operand staging: 16-byte slot permutation of an LDS row r of RB bytes
// (64-byte rows: (r >> 2) & 3; 128-byte rows: (r >> 1) & 7), applied on the
// global side of the LDS-DMA, and the byte offset within the tile of the
// 16-byte unit that lane `lane` fetches for stage row r.
// ---------------------------------------------------------------------------
template <int RB>
KD_HD constexpr int swz(int r) {
  static_assert(RB == 64 || RB == 128, "row bytes");
  return RB == 64 ? ((r >> 2) & 3) : ((r >> 1) & 7);
}
template <int RB>
KD_HD constexpr uint32_t dma_src_offset(int r, int lane, int64_t stride_bytes) {
  return (uint32_t)(r * stride_bytes + (((lane % (RB / 16)) ^ swz<RB>(r)) << 4));
}

// ---------------------------------------------------------------------------
// Teacher-id hit lists: an entry of the list of the wave tile holding
// z[t, v] codes (v % kHitV, t % kHitT) in 13 bits.
// ---------------------------------------------------------------------------
KD_HD constexpr uint32_t hit_code(int v, int t) {   // v, t >= 0
  return (((uint32_t)v % (uint32_t)kHitV) << 6) | ((uint32_t)t % (uint32_t)kHitT);
}
KD_HD constexpr int hit_code_v(uint32_t h) { return (int)(h >> 6); }
KD_HD constexpr int hit_code_t(uint32_t h) { return (int)(h & 63u); }

// ---------------------------------------------------------------------------
// Head-gradient epilogue (fp32 grad_W read-modify-write through a buffer
// resource per wave, 32-bit offsets).  The resource starts at row m0 and
// spans accum_rows(m0, nrows, M) rows of ld floats; a lane whose column is
// past N gets an offset beyond every resource.
// ---------------------------------------------------------------------------
constexpr uint32_t kOutside = 0x80000000u;
KD_HD constexpr int accum_rows(int m0, int nrows, int M) { return imax(0, imin(nrows, M - m0)); }
// offset of column n in the lane's first accumulator row (acc_row(0, lane))
KD_HD constexpr uint32_t accum_lane_offset(int n, int N, int lane, uint32_t ld4) {
  return n < N ? (uint32_t)(4 * (lane >> 5)) * ld4 + (uint32_t)n * 4u : kOutside;
}
// register r of the lane's 32-row tile i
KD_HD constexpr uint32_t accum_elem_offset(uint32_t lane_off, int i, int r, uint32_t ld4) {
  return lane_off + (uint32_t)(acc_row(r, 0) + 32 * i) * ld4;
}
// 64 x 160 wave tiles: columns 96..159 staged in LDS as [64][kWideStride]
// floats (rows of 288 bytes) and updated with 16-byte accesses
constexpr int kWideStride = 72;
KD_HD constexpr int wide_stage_index(int i, int j, int r, int lane) {   // j = 3 or 4
  return (32 * i + acc_row(r, lane)) * kWideStride + 32 * (j - 3) + acc_col(lane);
}
KD_HD constexpr int wide_read_row(int q, int lane) { return 4 * q + (lane >> 4); }
KD_HD constexpr int wide_read_col(int lane) { return 4 * (lane & 15); }
KD_HD constexpr uint32_t wide_lane_offset(int n, int N, int lane, uint32_t ld4) {
  return n < N ? (uint32_t)(lane >> 4) * ld4 + (uint32_t)n * 4u : kOutside;
}
KD_HD constexpr uint32_t wide_elem_offset(uint32_t lane_off, int q, uint32_t ld4) {
  return lane_off + (uint32_t)(4 * q) * ld4;
}

// ---------------------------------------------------------------------------
// Gradient epilogue staging (bf16, 128 x 64 wave tiles, 16 KB of LDS per
// wave, used once per layout).
//   G   [64 t][128 v]: 256-byte rows; 16-byte slot u of row t at u ^ (t & 15)
//   G^T [128 v][64 t]: 128-byte rows; 64-byte halves swapped on rows with
//                      bit 2 set
// ---------------------------------------------------------------------------
// 8-byte write of v = vl0 .. vl0 + 3 (vl0 a multiple of 4) of row tl
KD_HD constexpr int g_stage_offset(int tl, int vl0) {
  return tl * 256 + (((vl0 >> 3) ^ (tl & 15)) << 4) + ((vl0 & 7) << 1);
}
// 16-byte read q of a lane: row g_read_row, v = 8 * g_read_unit .. + 7
KD_HD constexpr int g_read_row(int q, int lane) { return 4 * q + (lane >> 4); }
KD_HD constexpr int g_read_unit(int lane) { return lane & 15; }
KD_HD constexpr int g_read_offset(int q, int lane) {
  return g_read_row(q, lane) * 256 + ((g_read_unit(lane) ^ (g_read_row(q, lane) & 15)) << 4);
}
// 2-byte write of (v = vl, t = tl)
KD_HD constexpr int gt_stage_offset(int vl, int tl) { return vl * 128 + ((tl * 2) ^ (((vl >> 2) & 1) << 6)); }
// 16-byte read q of a lane: row gt_read_row, t = 8 * gt_read_unit .. + 7
KD_HD constexpr int gt_read_row(int q, int lane) { return 8 * q + (lane >> 3); }
KD_HD constexpr int gt_read_unit(int lane) { return lane & 7; }
KD_HD constexpr int gt_read_offset(int q, int lane) {
  return gt_read_row(q, lane) * 128 + ((gt_read_unit(lane) * 16) ^ (((gt_read_row(q, lane) >> 2) & 1) << 6));
}
constexpr int kGradStageBytes = 16384;

// ---------------------------------------------------------------------------
// Cache builder: the GEMM epilogue stores the chunk's logits z[t][v] (rows of
// ldz floats, ldz a multiple of 256) through 16 KB of LDS per wave, one
// 32-column half of its 128 x 64 tile at a time, staged as [32 t][128 v]
// fp32: 512-byte rows, 16-byte unit u of row t at u ^ t.
// ---------------------------------------------------------------------------
// byte offset of the 16-byte write of v = vl0 .. vl0 + 3 (vl0 a multiple of 4) of row tl
KD_HD constexpr int cz_stage_offset(int tl, int vl0) { return tl * 512 + (((vl0 >> 2) ^ tl) << 4); }
// 16-byte read q of a lane: row cz_read_row, v = 4 * cz_read_unit .. + 3
KD_HD constexpr int cz_read_row(int q, int lane) { return 2 * q + (lane >> 5); }
KD_HD constexpr int cz_read_unit(int lane) { return lane & 31; }
KD_HD constexpr int cz_read_offset(int q, int lane) {
  return cz_read_row(q, lane) * 512 + ((cz_read_unit(lane) ^ cz_read_row(q, lane)) << 4);
}
// element offset in z of that read's four values: row n, columns m0 + 4 unit ..
KD_HD constexpr int64_t cz_global_offset(int n, int64_t ldz, int m0, int unit) {
  return (int64_t)n * ldz + m0 + 4 * unit;
}
constexpr int kCacheStageBytes = 16384;

// ---------------------------------------------------------------------------
// Teacher rows: LDS of kl_rows_kernel and teacher_p_kernel (Kp 64-bit sort
// keys, Kp the power of two >= K, then K floats).
// ---------------------------------------------------------------------------
KD_HD constexpr int teacher_sort_len(int K) {
  int p = 1;
  while (p < K) p <<= 1;
  return p;
}
KD_HD constexpr size_t teacher_lds_bytes(int K) { return (size_t)teacher_sort_len(K) * 8 + (size_t)K * 4; }

}  // namespace kd
