// Sustained MFMA ceiling probe (measurement only; not part of the loss).
//
// The bf16 datasheet peak assumes the 2.4 GHz shader clock.  With random
// operands the MFMA datapath alone holds the chip at its power limit, where
// the clock is lower, so the GEMMs are also compared against what the MFMA
// pipes deliver with no memory traffic at all: every wave issues
// v_mfma_f32_32x32x16_bf16 back to back on register operands, in the
// GEMM's own wave shape (a 4 x 2 grid of 32x32 accumulator tiles, 8 waves
// per 512-thread block) and cycling through 8 A and 4 B fragments so the
// operands change from one instruction to the next as they do in a GEMM.
#pragma once
#include "kd_gemm.hpp"

namespace kd {

__device__ __forceinline__ uint32_t probe_hash(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// two bf16 values uniform in [-1, 1) (or zeros)
__device__ __forceinline__ uint32_t probe_pair(uint32_t s, bool zero) {
  if (zero) return 0u;
  const uint32_t h = probe_hash(s);
  const float a = (float)(h & 0xffffu) * (1.f / 32768.f) - 1.f, b = (float)(h >> 16) * (1.f / 32768.f) - 1.f;
  return pack_bf16x2(a, b);
}

// out[thread] = sum of the thread's accumulators (keeps the MFMAs live);
// 64 MFMAs of 32768 FLOPs per wave and iteration.
__global__ __launch_bounds__(512) void mfma_probe_kernel(int iters, int zero, float* out) {
  const uint32_t gid = blockIdx.x * blockDim.x + threadIdx.x;
  u32x4 fa[8], fb[4];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t s = gid * 64u + 4u * i;
    fa[i] = u32x4{probe_pair(s, zero), probe_pair(s + 1, zero), probe_pair(s + 2, zero), probe_pair(s + 3, zero)};
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t s = gid * 64u + 32u + 4u * j;
    fb[j] = u32x4{probe_pair(s, zero), probe_pair(s + 1, zero), probe_pair(s + 2, zero), probe_pair(s + 3, zero)};
  }
  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int q = 0; q < 8; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) mfma_group<Bf16>(acc[i][j], fa[(i + q) & 7], fb[(j + q) & 3]);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) s += acc[i][j][r];
  out[gid] = s;
}

}  // namespace kd
