// kd_cache.hpp -- kernels of the offline top-K teacher-logit cache builder
// (gfx950): for every row t of the teacher's final hidden states, the K
// largest logits z[t, v] = h_t . W_v over the whole vocabulary, with their
// ids, in descending order (equal logits: lower id first).  The teacher runs
// once and this record replaces it during training (Glonce, "Multiverse
// Computing cuts LLM distillation VRAM by 15x with chunked KL loss",
// paragraph on Multiverse's two-part fix; ainewsbank.com, "Multiverse
// Computing Tests Lower-Memory Long-Context Distillation", section "Two
// changes remove different bottlenecks").
//
// Per chunk of rows, with the same GEMM as the loss:
//   GEMM    z^T = W H_c^T; the epilogue keeps, per 32-row vocabulary block
//           and row, the block's largest logit, and stores the chunk's fp32
//           logits row by row (EpiBlockMax);
//   select  per row, the K-th largest of those block maxima: a lower bound
//           theta_t such that at least K logits are >= theta_t (K of the
//           blocks have their maximum >= it); radix select on order-
//           preserving keys (cache_threshold_kernel);
//   collect one streaming pass over the stored logits appends every
//           z >= theta_t of row t to the row's candidate list
//           (cache_collect_kernel);
//   sort    per row, the candidates by (z descending, id ascending), the
//           first K written out (cache_select_kernel).
// Keeping the chunk's logits (chunk x V fp32) costs one HBM write and one
// read of them where a second GEMM pass would cost as much MFMA work as the
// first.
// Rows with more candidates than the list holds (many logits tied at or
// above theta_t) are redone exactly by cache_fallback_kernel, which streams
// the vocabulary through a sorted top-K in LDS with its own dot products.
#pragma once

#include "kd_kernels.hpp"

namespace kd {

// Order-preserving unsigned keys of fp32 values (larger float, larger key).
__device__ __forceinline__ uint32_t fkey(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float fkey_inv(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}
// Sort key of a candidate: z descending, then id ascending, as one uint64
// (larger = earlier).
__device__ __forceinline__ uint64_t cand_key(float z, uint32_t id) {
  return ((uint64_t)fkey(z) << 32) | (uint64_t)(0xffffffffu - id);
}


// The GEMM's epilogue: per 32-row vocabulary block and column (row t), the
// largest logit of the block's valid rows, stored per row t: out[t][block];
// and the tile's logits, stored as z[t][v] (rows of ldz floats; entries at
// v >= V hold padding and are never read).  The logits go through the
// wave's 16 KB of the freed LDS ring, one 32-column half at a time, so that
// they leave as 16-byte non-temporal stores of whole 512-byte row segments.
struct EpiBlockMax {
  float* out;   // [rows][ldb]: row t's block maxima contiguous
  int ldb;      // V_p / 32 (a multiple of 8)
  int V;
  float* z;     // [R_p][ldz] the chunk's logits
  int64_t ldz;  // V_p

  template <int FM, int FN>
  __device__ __forceinline__ void apply(f32x16 (&acc)[FM][FN], const EpiCtx& c) const {
    static_assert(FM == 4, "a wave strip holds four 32-row blocks (one 16-byte store per row)");
    const int rows_valid = V - c.m0;
    if (rows_valid <= 0) return;                    // no valid row here (never read)
    if (rows_valid < FM * 32) clamp_padding_rows<FM, FN>(acc, rows_valid, c.lane);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int n = c.n0 + 32 * j + acc_col(c.lane);
      float mx[FM];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        float m = acc[i][j][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) m = fmaxf(m, acc[i][j][r]);
        mx[i] = fmaxf(m, __shfl_xor(m, 32));
      }
      // lane < 32: column (row t) n, blocks m0/32 .. +3
      if (c.lane < 32) *(f32x4*)(out + (int64_t)n * ldb + c.m0 / kBlockRows) = f32x4{mx[0], mx[1], mx[2], mx[3]};
      store_half(acc, j, c);
    }
  }

  // columns 32 j .. 32 j + 31 of the wave's tile: staged [32 t][128 v], then
  // each read of a lane is 4 consecutive v of one row, and 32 lanes store a
  // row's 512 bytes (the wave's LDS operations run in order, so the second
  // half's writes follow the first half's reads)
  template <int FM, int FN>
  __device__ __forceinline__ void store_half(f32x16 (&acc)[FM][FN], int j, const EpiCtx& c) const {
    static_assert(FM == 4, "128-row strips");
    char* lds = c.smem + c.wid * (c.smem_bytes / c.nwaves);
    const int tl = acc_col(c.lane);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        *(f32x4*)(lds + cz_stage_offset(tl, 32 * i + 8 * g4 + 4 * (c.lane >> 5))) =
            f32x4{acc[i][j][4 * g4], acc[i][j][4 * g4 + 1], acc[i][j][4 * g4 + 2], acc[i][j][4 * g4 + 3]};
    __builtin_amdgcn_s_waitcnt(0xC07F);             // lgkmcnt(0): the wave's staging writes are done
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const f32x4 val = *(const f32x4*)(lds + cz_read_offset(q, c.lane));
      __builtin_nontemporal_store(
          val, (f32x4*)(z + cz_global_offset(c.n0 + 32 * j + cz_read_row(q, c.lane), ldz, c.m0, cz_read_unit(c.lane))));
    }
  }
};

// Inclusive prefix sum over the 256 threads of a block (4 waves).
__device__ __forceinline__ int block_incl_scan_256(int v, int* s_w) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o);
    if (lane >= o) v += u;
  }
  if (lane == 63) s_w[w] = v;
  __syncthreads();
  int add = 0;
  for (int i = 0; i < w; ++i) add += s_w[i];
  __syncthreads();
  return v + add;
}

// theta_t = the K-th largest of the row's nbv valid block maxima (MSB-first
// radix select over 8-bit digits of the order-preserving keys), or -inf when
// there are fewer than K blocks (then every logit is a candidate).  One
// block of 256 threads per row; the row's maxima are read contiguously, each
// wave counts into its own histogram, and the digit holding the rank is
// found with a block-wide prefix sum over the bins in descending order.
__global__ __launch_bounds__(256) void cache_threshold_kernel(const float* bmax, int ldb, int nbv, int K,
                                                              float* theta) {
  __shared__ int hist[4][256];
  __shared__ int s_w[4];
  __shared__ uint32_t s_prefix;
  __shared__ int s_k;
  const int t = blockIdx.x, tid = threadIdx.x, wave = tid >> 6;
  if (nbv < K) {
    if (tid == 0) theta[t] = -INFINITY;
    return;
  }
  const float* row = bmax + (int64_t)t * ldb;
  uint32_t prefix = 0, mask = 0;
  int k = K;                                        // rank still to find among the matching keys
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 4 * 256; i += 256) (&hist[0][0])[i] = 0;
    __syncthreads();
    for (int i = tid; i < nbv; i += 256) {
      const uint32_t key = fkey(row[i]);
      if ((key & mask) == prefix) atomicAdd(&hist[wave][(key >> shift) & 255], 1);
    }
    __syncthreads();
    const int b = 255 - tid;                         // bins in descending order
    const int cnt = hist[0][b] + hist[1][b] + hist[2][b] + hist[3][b];
    const int incl = block_incl_scan_256(cnt, s_w);  // keys in bins >= b
    if (incl >= k && incl - cnt < k) {               // exactly one bin holds rank k
      s_prefix = prefix | ((uint32_t)b << shift);
      s_k = k - (incl - cnt);
    }
    __syncthreads();
    prefix = s_prefix;
    k = s_k;
    mask |= 255u << shift;
  }
  if (tid == 0) theta[t] = fkey_inv(prefix);
}

// Collect: every valid z >= theta_t of row t of the stored logits goes to
// the row's candidate list (cand[t][0, cap), count cnt[t]; appends past cap
// only count).  One block per row streams the row's V floats with 16-byte
// loads, four per thread in flight.
__global__ __launch_bounds__(256) void cache_collect_kernel(const float* z, int64_t ldz, int V, const float* theta,
                                                            int* cnt, uint2* cand, int cap) {
  __shared__ int s_n;
  const int t = blockIdx.x;
  if (threadIdx.x == 0) s_n = 0;
  __syncthreads();
  const float th = theta[t];
  const float* row = z + (int64_t)t * ldz;
  uint2* out = cand + (int64_t)t * cap;
  // ldz is a multiple of 256 >= V: every 16-byte load that starts below V
  // stays inside the row
  for (int v0 = 4 * (int)threadIdx.x; v0 < V; v0 += 4 * 4 * 256) {
    f32x4 q[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int v = v0 + u * 4 * 256;
      q[u] = v < V ? __builtin_nontemporal_load((const f32x4*)(row + v)) : f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int v = v0 + u * 4 * 256 + e;
        if (v < V && q[u][e] >= th) {
          const int pos = atomicAdd(&s_n, 1);
          if (pos < cap) out[pos] = make_uint2(__float_as_uint(q[u][e]), (uint32_t)v);
        }
      }
  }
  __syncthreads();
  if (threadIdx.x == 0) cnt[t] = s_n;
}

// In-LDS bitonic sort of n (a power of two) uint64 keys, descending.
__device__ __forceinline__ void bitonic_desc(uint64_t* s, int n) {
  for (int size = 2; size <= n; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < (n >> 1); i += blockDim.x) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool desc = ((lo & size) == 0);
        const uint64_t a = s[lo], b = s[hi];
        if ((a < b) == desc) {
          s[lo] = b;
          s[hi] = a;
        }
      }
      __syncthreads();
    }
  }
}

// Per row: sort the candidates, write the first K (ids, logits); rows whose
// list overflowed are marked for the exact fallback (ovf[t] = 1) and left to
// it.  cap is a power of two; dynamic LDS holds cap keys.
__global__ __launch_bounds__(256) void cache_select_kernel(const int* cnt, const uint2* cand, int cap, int K,
                                                           int32_t* out_idx, float* out_logit, int* ovf) {
  extern __shared__ uint64_t s_keys[];
  const int t = blockIdx.x;
  const int n = cnt[t];
  if (n > cap) {
    if (threadIdx.x == 0) ovf[t] = 1;
    return;
  }
  if (threadIdx.x == 0) ovf[t] = 0;
  int m = 1;
  while (m < n) m <<= 1;
  for (int i = threadIdx.x; i < m; i += blockDim.x) {
    uint64_t key = 0;                               // padding sorts last
    if (i < n) {
      const uint2 e = cand[(int64_t)t * cap + i];
      key = cand_key(__uint_as_float(e.x), e.y);
    }
    s_keys[i] = key;
  }
  __syncthreads();
  bitonic_desc(s_keys, m);
  for (int k = threadIdx.x; k < K; k += blockDim.x) {
    const uint64_t key = s_keys[k];
    out_idx[(int64_t)t * K + k] = (int32_t)(0xffffffffu - (uint32_t)key);
    out_logit[(int64_t)t * K + k] = fkey_inv((uint32_t)(key >> 32));
  }
}

// Exact fallback for marked rows: the row's logits recomputed by plain dot
// products (fp32, summed along d), streamed in batches of kFbBatch ids
// through a sorted top-K kept in LDS.  Slow (a full pass over W per row);
// it runs only for rows with more tied candidates than the list holds.

template <class E>
__global__ __launch_bounds__(256) void cache_fallback_kernel(const typename E::T* H, int64_t ldh,
                                                             const typename E::T* W, int64_t ldw, int d, int V, int K,
                                                             int half, const int* ovf, int32_t* out_idx,
                                                             float* out_logit) {
  // s_keys: 2 * half keys; [0, half) the best so far (half: a power of two
  // >= max(K, kFbBatch)), [half, 2 half) the next batch and zero padding
  extern __shared__ uint64_t s_keys[];
  const int t = blockIdx.x;
  if (!ovf[t]) return;
  const int tot = 2 * half;
  for (int i = threadIdx.x; i < half; i += blockDim.x) s_keys[i] = 0;
  const typename E::T* h = H + (int64_t)t * ldh;
  for (int v0 = 0; v0 < V; v0 += kFbBatch) {
    for (int i = threadIdx.x; i < half; i += blockDim.x) {
      const int v = v0 + i;
      uint64_t key = 0;
      if (i < kFbBatch && v < V) {
        const typename E::T* w = W + (int64_t)v * ldw;
        float z = 0.f;
        for (int j = 0; j < d; ++j) z += load_elem<E>(h + j) * load_elem<E>(w + j);
        key = cand_key(z, (uint32_t)v);
      }
      s_keys[half + i] = key;
    }
    __syncthreads();
    bitonic_desc(s_keys, tot);                      // the best `half` move to the front
  }
  for (int k = threadIdx.x; k < K; k += blockDim.x) {
    const uint64_t key = s_keys[k];
    out_idx[(int64_t)t * K + k] = (int32_t)(0xffffffffu - (uint32_t)key);
    out_logit[(int64_t)t * K + k] = fkey_inv((uint32_t)(key >> 32));
  }
}

}  // namespace kd
