// kd_kernels.hpp -- epilogues of the shared GEMM and the small kernels of the
// fused chunked top-K KL loss (gfx950).
//
// Notation: a chunk holds rows t in [0, R) of the sequence (global row
// c0 + t); S = z / tau; statistics over the vocabulary are kept in base 2,
// x2 = z * log2(e) / tau, so that exp2 / log2 map to v_exp_f32 / v_log_f32.
#pragma once

#include "kd_gemm.hpp"
#include <math.h>

namespace kd {

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// GEMM epilogues
// ---------------------------------------------------------------------------

// Rows of a wave's strip at or past `rows_valid` (vocabulary padding, whose
// logits are exactly 0 because their A rows read as zeros) are pushed to
// about -1e38 so that they vanish from maxima and from sums of exp2.  The
// clamp is arithmetic (no per-element predicate), so it costs a few VALU
// operations per element on every tile and keeps no lane masks alive.
template <int FM, int FN>
__device__ __forceinline__ void clamp_padding_rows(f32x16 (&acc)[FM][FN], int rows_valid, int lane) {
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float lim = ((float)(rows_valid - 32 * i - acc_row(r, lane)) - 0.5f) * 1e38f;
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j][r] = fminf(acc[i][j][r], lim);
    }
}

// Forward pass of a chunk: per (vocabulary strip of one wave, row t) the
// running max and sum of exp2 -- the partial logsumexp that the online merge
// folds into the row's full-vocabulary normaliser.  The logits themselves are
// never written: each chunk contributes its reductions to the loss and is
// then dropped (Glonce, "Multiverse Computing cuts LLM distillation VRAM by
// 15x with chunked KL loss", paragraph on Multiverse's two-part fix).
//
// The same epilogue also picks out the logits at the teacher's cached ids:
// every (t, k) of the chunk is filed beforehand (hit_build_kernel) under the wave
// sub-tile that holds z[t, idx[t,k]], and the wave copies those values from
// its accumulators to zsel[t*K + k].  The top-K gather of the KL thus reads
// no W rows.

struct EpiLsePartial {
  float2* part;   // [nvt][ldp]: (max x2, sum exp2(x2 - max)) per strip and row
  int ldp;
  int V;
  float c2;       // log2(e) / tau
  const int* hit_off;   // [nvt * nbt + 1] start of each wave tile's hit list
  const uint2* hits;    // (slot t*K + k, (v % kHitV) << 6 | (t % kHitT))
  float* zsel;          // [R * K] z at the teacher ids
  int hstride;          // offsets per row group: strips + 1

  // The wave tile's hit-list bounds (step 0) and its first 64 entries
  // (step 1) are loaded during the main loop.
  static constexpr int kPrefetchSteps = 1;
  template <int FM, int FN>
  __device__ __forceinline__ void prefetch(EpiCtx& c, int step) const {
    // raw values only: computing on a value right after its load would
    // wait for it there
    if (step == 0) {
      const int b = (c.n0 / kHitT) * hstride + c.m0 / kHitV;
      c.pf[0] = (uint32_t)hit_off[b];
      c.pf[1] = (uint32_t)hit_off[b + 1];
    } else {
      const int e0 = (int)c.pf[0];
      c.pf[1] -= c.pf[0];
      const uint2 hv = c.lane < (int)c.pf[1] ? hits[e0 + c.lane] : make_uint2(0u, 0u);
      c.pf[2] = hv.x;
      c.pf[3] = hv.y;
    }
  }

  template <int FM, int FN>
  __device__ __forceinline__ void apply(f32x16 (&acc)[FM][FN], const EpiCtx& c) const {
    static_assert(FM * 32 == kHitV && FN * 32 == kHitT, "hit lists are filed by wave tile");
    const int vt = c.m0 / (FM * 32);
    {
      // the wave's entries, up to 64 per vector load (the first 64 loaded
      // ahead), then one at a time from registers
      const int e0 = (int)c.pf[0], n = (int)c.pf[1];
      for (int base = 0; base < n; base += 64) {
        const uint2 hv = base == 0 ? make_uint2(c.pf[2], c.pf[3])
                                   : (base + c.lane < n ? hits[e0 + base + c.lane] : make_uint2(0u, 0u));
        const int cnt = min(64, n - base);
        for (int q = 0; q < cnt; ++q) {
          const uint32_t hx = (uint32_t)__builtin_amdgcn_readlane((int)hv.x, q);
          const uint32_t hy = (uint32_t)__builtin_amdgcn_readlane((int)hv.y, q);
          const int vl = hit_code_v(hy), tl = hit_code_t(hy);
          const int r = acc_reg_of(vl & 31);                   // register and lane holding that element
          const int owner = acc_lane_of(vl & 31, tl);
          float z = 0.f;
#pragma unroll
          for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
              if (i == (vl >> 5) && j == (tl >> 5)) z = acc[i][j][r];
          if (c.lane == owner) zsel[hx] = z;
        }
      }
    }
    const int rows_valid = V - c.m0;          // vocabulary rows of this strip that exist
    if (rows_valid <= 0) {                    // strip entirely in the padding
#pragma unroll
      for (int j = 0; j < FN; ++j)
        if (c.lane < 32) part[(int64_t)vt * ldp + c.n0 + 32 * j + c.lane] = make_float2(-INFINITY, 0.f);
      return;
    }
    if (rows_valid < FM * 32) clamp_padding_rows<FM, FN>(acc, rows_valid, c.lane);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc[i][j][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32)) * c2;   // c2 > 0: max commutes with the scaling
      float sm = 0.f;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) sm += fast_exp2(acc[i][j][r] * c2 - mx);
      sm += __shfl_xor(sm, 32);
      if (c.lane < 32) part[(int64_t)vt * ldp + c.n0 + 32 * j + c.lane] = make_float2(mx, sm);
    }
  }
};

// Gradient scale g tau / N (0 when no position counts).
__device__ __forceinline__ float grad_scale(const int* count, const float* grad_loss, float tau) {
  const int N = *count;
  return N > 0 ? (grad_loss ? *grad_loss : 1.f) * (tau / (float)N) : 0.f;
}

// Mask byte read for every row when the caller passes no mask.
__device__ const uint8_t kMaskAll = 1;

// Backward recompute of a chunk: the logit gradient of the loss,
// G[t,v] = g (tau/N) m_t q[t,v] (g = dL/dloss from the caller, 1 in the
// fused call), written in two layouts (G [R_p][V_p] and G^T [V_p][R_p]) for
// the two gradient GEMMs; entries at v >= V are unused.  The sparse teacher
// part -g (tau/N) m_t P[t,v] is subtracted in the epilogue from the fp32
// values, through the chunk's hit lists, before G is rounded.
template <class E>
struct EpiGrad {
  typename E::T* G;
  int64_t ldg;
  typename E::T* Gt;
  int64_t ldgt;
  const float* lse;       // [R] row normaliser, times lse_to2 in base 2
  float lse_to2;          // 1 (base-2 input) or log2(e) (natural-log input)
  const uint8_t* mask;    // chunk rows, or nullptr
  const int* count;       // N
  const float* grad_loss; // device scalar g, or nullptr for 1
  float tau, c2;
  int V, R;
  // The sparse teacher part: the chunk's teacher-id hit lists and the
  // teacher probabilities psel[t*K + k] (hit_off == nullptr: left out).
  const int* hit_off;
  const uint2* hits;
  const float* psel;
  int hstride;

  // Loaded during the main loop (EpiCtx::pf): step 0 the count N, g, the
  // lane's columns' normalisers and mask bytes, and the hit-list bounds;
  // step 1 the first 64 hit entries; step 2 their teacher probabilities.
  //   pf: 0 e0, 1 end (n from step 1), 2-3 entry, 4 N, 5 g, 6+j lse,
  //       8+j mask byte, 10 p
  static constexpr int kPrefetchSteps = 2;
  template <int FM, int FN>
  __device__ __forceinline__ void prefetch(EpiCtx& c, int step) const {
    static_assert(FN <= 2, "two prefetched columns per lane");
    if (step == 0) {
      c.pf[4] = (uint32_t)*count;
      c.pf[5] = __builtin_bit_cast(uint32_t, grad_loss ? *grad_loss : 1.f);
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        // raw loaded values only, from clamped addresses (rows past the
        // chunk are zeroed in apply): a value that is computed on, or
        // merged from two branches, right after its load is waited for there
        const int nc = min(c.n0 + 32 * j + acc_col(c.lane), R - 1);
        c.pf[6 + j] = __builtin_bit_cast(uint32_t, lse[nc]);
        typedef const __attribute__((address_space(1))) uint8_t* GlobalByte;   // a global, not a flat, load
        c.pf[8 + j] = (uint32_t)*(mask ? (GlobalByte)(mask + nc) : (GlobalByte)&kMaskAll);
      }
      c.pf[0] = c.pf[1] = 0u;
      if (hit_off) {
        const int b = (c.n0 / kHitT) * hstride + c.m0 / kHitV;
        c.pf[0] = (uint32_t)hit_off[b];
        c.pf[1] = (uint32_t)hit_off[b + 1];
      }
    } else if (step == 1) {
      const int e0 = (int)c.pf[0];
      c.pf[1] -= c.pf[0];
      const uint2 hv = c.lane < (int)c.pf[1] ? hits[e0 + c.lane] : make_uint2(0u, 0u);
      c.pf[2] = hv.x;
      c.pf[3] = hv.y;
    } else {
      c.pf[10] = c.lane < (int)c.pf[1] ? __builtin_bit_cast(uint32_t, psel[c.pf[2]]) : 0u;
    }
  }

  template <int FM, int FN>
  __device__ __forceinline__ void apply(f32x16 (&acc)[FM][FN], const EpiCtx& c) const {
    // G values in fp32, in place: acc <- sc * q (sc = g tau m_t / N), formed
    // as one exp2 per element with |sc| folded into the exponent,
    // q |sc| = exp2(z c2 - (lse2 - log2 |sc|)), and the sign of g applied
    // after (it is the same for the whole call).  sc = 0 (masked rows, rows
    // past the chunk, N = 0, g = 0) gives an exponent of -inf, hence 0.
    const int N = (int)c.pf[4];
    const float s = N > 0 ? __builtin_bit_cast(float, c.pf[5]) * (tau / (float)N) : 0.f;
    float sc[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      // row scale (0 on masked rows and rows past the chunk) and base-2 normaliser
      const bool row = c.n0 + 32 * j + acc_col(c.lane) < R;
      sc[j] = row && c.pf[8 + j] ? s : 0.f;
      const float l2 = row ? __builtin_bit_cast(float, c.pf[6 + j]) * lse_to2 : 0.f;
      const float off = l2 - __log2f(fabsf(sc[j]));
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = fast_exp2(acc[i][j][r] * c2 - off);
    }
    if (s < 0.f) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] = -acc[i][j][r];
    }
    if (hit_off) sparse_part<FM, FN>(acc, sc, c);
    if constexpr (E::kBytes == 2 && FM == 4 && FN == 2) {
      if (c.smem_bytes / c.nwaves >= kStageBytes) {
        store_staged(acc, c);
        return;
      }
    }
    store_direct<FM, FN>(acc, c);
  }

  // -sc_t P at (v = idx[t,k], t) for every (t, k) filed under this wave
  // tile, where psel holds P once per (t, v) (repeated ids are merged by
  // merged_target_row, their later entries hold 0, so the order of the list
  // does not reach the result); the lane that holds the element applies it,
  // so G is rounded once.
  template <int FM, int FN>
  __device__ __forceinline__ void sparse_part(f32x16 (&acc)[FM][FN], const float (&sc)[FN], const EpiCtx& c) const {
    static_assert(FM * 32 == kHitV && FN * 32 == kHitT, "hit lists are filed by wave tile");
    const int e0 = (int)c.pf[0], n = (int)c.pf[1];
    for (int base = 0; base < n; base += 64) {
      // up to 64 entries and their p per vector load (the first 64 loaded
      // ahead), then one at a time
      const bool in = base + c.lane < n;
      uint2 hv;
      float pv;
      if (base == 0) {
        hv = make_uint2(c.pf[2], c.pf[3]);
        pv = __builtin_bit_cast(float, c.pf[10]);
      } else {
        hv = in ? hits[e0 + base + c.lane] : make_uint2(0u, 0u);
        pv = in ? psel[hv.x] : 0.f;
      }
      const int cnt = min(64, n - base);
      for (int q = 0; q < cnt; ++q) {
        const uint32_t hy = (uint32_t)__builtin_amdgcn_readlane((int)hv.y, q);
        const float p = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, pv), q));
        const int vl = hit_code_v(hy), tl = hit_code_t(hy);
        const int r = acc_reg_of(vl & 31);                   // register and lane holding that element
        const int owner = acc_lane_of(vl & 31, tl);
        if (c.lane == owner) {
#pragma unroll
          for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
              if (i == (vl >> 5) && j == (tl >> 5)) acc[i][j][r] -= sc[j] * p;
        }
      }
    }
  }

  // Rows past the vocabulary (z = 0 from zero-filled A rows) get finite junk
  // in both store paths (|sc| 2^-lse2): the head-gradient GEMM never reads
  // G^T rows >= V, and the hidden-gradient GEMM multiplies G's columns >= V
  // by the zero columns of the padded W^T.
  template <int FM, int FN>
  __device__ __forceinline__ void store_direct(f32x16 (&acc)[FM][FN], const EpiCtx& c) const {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int n = c.n0 + 32 * j + acc_col(c.lane);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int v0 = c.m0 + 32 * i + 8 * g4 + 4 * (c.lane >> 5);
          float gv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) gv[e] = acc[i][j][4 * g4 + e];
          store4(G + (int64_t)n * ldg + v0, gv);
#pragma unroll
          for (int e = 0; e < 4; ++e) Gt[(int64_t)(v0 + e) * ldgt + n] = store_cvt<E>(gv[e]);
        }
    }
  }

  // bf16 with 128 x 64 wave tiles: the wave's tile goes through its own
  // 16 KB of the (now free) LDS ring twice, once per layout, so that both
  // layouts leave as 16-byte stores of whole 128/256-byte row segments
  // instead of 8-byte and 2-byte scattered stores (0.05-0.07 ms less per
  // launch on the 32K workload's recompute GEMM).  The stores are
  // non-temporal: the 1.6 GB a launch writes is read back only by later
  // GEMMs, far beyond what the caches hold (another ~0.05 ms per launch).
  //   G staging  [64 t][128 v], 256-byte rows, 16-byte slot u of row t at
  //              u ^ (t & 15) (the 8-byte writes of a half-wave, 32 rows
  //              apart by 256 bytes, spread over the banks);
  //   G^T staging [128 v][64 t], 128-byte rows, 64-byte halves swapped on
  //              rows with bit 2 set (the two half-waves write rows 4 apart).
  static constexpr int kStageBytes = kGradStageBytes;

  __device__ __forceinline__ void store_staged(f32x16 (&acc)[4][2], const EpiCtx& c) const {
    char* lds = c.smem + c.wid * (c.smem_bytes / c.nwaves);
    uint2 pk[4][2][4];   // bf16 values, 4 consecutive v per entry
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int tl = 32 * j + acc_col(c.lane);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int vl0 = 32 * i + 8 * g4 + 4 * (c.lane >> 5);
          pk[i][j][g4] = make_uint2(pack_bf16x2(acc[i][j][4 * g4], acc[i][j][4 * g4 + 1]),
                                    pack_bf16x2(acc[i][j][4 * g4 + 2], acc[i][j][4 * g4 + 3]));
          *(uint2*)(lds + g_stage_offset(tl, vl0)) = pk[i][j][g4];
        }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);       // lgkmcnt(0): the wave's staging writes are done
    // G: 64 rows x 16 slots; lane -> row 4q + lane/16, slot lane % 16
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int t = g_read_row(q, c.lane), u = g_read_unit(c.lane);
      const u32x4 val = *(const u32x4*)(lds + g_read_offset(q, c.lane));
      __builtin_nontemporal_store(val, (u32x4*)(G + (int64_t)(c.n0 + t) * ldg + c.m0 + 8 * u));
    }
    // G^T staging (the wave's LDS operations run in order: the reads above
    // see the old contents)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int tl = 32 * j + acc_col(c.lane);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int vl0 = 32 * i + 8 * g4 + 4 * (c.lane >> 5);
          const uint32_t h[4] = {pk[i][j][g4].x & 0xffffu, pk[i][j][g4].x >> 16, pk[i][j][g4].y & 0xffffu,
                                 pk[i][j][g4].y >> 16};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int vl = vl0 + e;
            *(uint16_t*)(lds + gt_stage_offset(vl, tl)) = (uint16_t)h[e];
          }
        }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);
    // G^T: 128 rows x 8 slots; lane -> row 8q + lane/8, slot lane % 8
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int v = gt_read_row(q, c.lane), u = gt_read_unit(c.lane);
      const u32x4 val = *(const u32x4*)(lds + gt_read_offset(q, c.lane));
      __builtin_nontemporal_store(val, (u32x4*)(Gt + (int64_t)(c.m0 + v) * ldgt + c.n0 + 8 * u));
    }
  }

  __device__ __forceinline__ static void store4(uint16_t* p, const float* g) {
    uint2 w;
    w.x = pack_bf16x2(g[0], g[1]);
    w.y = pack_bf16x2(g[2], g[3]);
    *(uint2*)p = w;
  }
  __device__ __forceinline__ static void store4(float* p, const float* g) {
    *(float4*)p = make_float4(g[0], g[1], g[2], g[3]);
  }
};

// Split-K partial of the hidden gradient: plain fp32 tile store into
// out[split][m][n] (the partials are summed in a fixed order afterwards).
struct EpiStoreSplit {
  float* out;
  int64_t ld;
  int64_t split_stride;

  template <int FM, int FN>
  __device__ __forceinline__ void apply(f32x16 (&acc)[FM][FN], const EpiCtx& c) const {
    float* base = out + (int64_t)c.split * split_stride;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = c.m0 + 32 * i + acc_row(r, c.lane);
          const int n = c.n0 + 32 * j + acc_col(c.lane);
          base[(int64_t)m * ld + n] = acc[i][j][r];
        }
  }
};

// Head gradient: grad_W[v][j] (+)= tile, accumulated across chunks in fp32
// (the first chunk stores).  grad_W (2.3 GB at V = 201088, d = 2880) is
// streamed once per launch, so its loads and stores are non-temporal.
//
// A wave reaches its 64 rows of grad_W through a buffer resource that ends
// at row M, with 32-bit offsets: rows past M read zeros and are not written,
// and a lane whose column is past N gets an offset beyond any resource, so
// the update needs neither predicates nor 64-bit address arithmetic per
// element (the host limits d to 2^20, so a wave's 64 rows span under 2^28
// bytes and no offset wraps).
struct EpiAccum {
  float* out;
  int64_t ld;
  int M, N;
  int first;

  static constexpr int kNT = 2;                       // non-temporal cache policy

  // (m0 is the same on every lane of a wave; readfirstlane says so to the
  // compiler, which keeps the resource in scalar registers)
  __device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(int m0, int nrows) const {
    const int m0u = __builtin_amdgcn_readfirstlane(m0);
    const int rows = accum_rows(m0u, nrows, M);
    const int bytes = __builtin_amdgcn_readfirstlane(rows * (int)ld * 4);
    return make_rsrc(out + (int64_t)m0u * ld, (uint32_t)bytes);
  }

  template <int FM, int FN>
  __device__ __forceinline__ void apply(f32x16 (&acc)[FM][FN], const EpiCtx& c) const {
    if constexpr (FM == 2 && FN == 5) {
      apply_wide(acc, c);
      return;
    }
    const __amdgpu_buffer_rsrc_t rs = rows_rsrc(c.m0, FM * 32);
    const uint32_t ld4 = (uint32_t)ld * 4u;
    // lane offset of column n in the lane's first row (acc_row(0, lane))
    uint32_t vo[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) vo[j] = accum_lane_offset(c.n0 + 32 * j + acc_col(c.lane), N, c.lane, ld4);
    // old values first (one burst of loads), then the stores
    if (!first) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            acc[i][j][r] += __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                rs, accum_elem_offset(vo[j], i, r, ld4), 0, kNT));
    }
    // (__float_as_uint takes the element by value; hipcc's __builtin_bit_cast
    // of a vector-element lvalue reads element 0 instead)
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i][j][r]), rs,
                                                accum_elem_offset(vo[j], i, r, ld4), 0, kNT);
  }

  // 64 x 160 wave tiles (256 x 320 blocks, 18 KB of the freed LDS ring per
  // wave).  Keeping all 160 old values of a lane in flight next to its 160
  // accumulators would not fit the registers, so columns 96..159 of the
  // wave's tile go through LDS and are updated with 16-byte accesses, while
  // columns 0..95 are updated straight from the accumulators.  Requires N
  // and ld multiples of 4 and a 16-byte aligned `out` (checked by the host).
  // (kWideStride = 72 floats per staged row: 288 B, so the two half-waves,
  // rows 4 apart, hit disjoint banks)
  __device__ __forceinline__ void apply_wide(f32x16 (&acc)[2][5], const EpiCtx& c) const {
    float* st = (float*)(c.smem + c.wid * (c.smem_bytes / c.nwaves));   // [64][72]
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 3; j < 5; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          st[wide_stage_index(i, j, r, c.lane)] = acc[i][j][r];
    const __amdgpu_buffer_rsrc_t rs = rows_rsrc(c.m0, 64);
    const uint32_t ld4 = (uint32_t)ld * 4u;
    // columns 0..95 from the accumulators: all old values in flight, then the stores
    uint32_t vo[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) vo[j] = accum_lane_offset(c.n0 + 32 * j + acc_col(c.lane), N, c.lane, ld4);
    if (!first) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 3; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            acc[i][j][r] += __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                rs, accum_elem_offset(vo[j], i, r, ld4), 0, kNT));
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 3; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i][j][r]), rs,
                                                accum_elem_offset(vo[j], i, r, ld4), 0, kNT);
    // columns 96..159 from LDS: lane -> row 4q + lane/16, columns 4 (lane % 16) .. +3
    __builtin_amdgcn_s_waitcnt(0xC07F);       // lgkmcnt(0): the wave's staging writes are done
    f32x4 v[16];
    const int col = wide_read_col(c.lane);
    const uint32_t vs = wide_lane_offset(c.n0 + 96 + col, N, c.lane, ld4);
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      v[q] = *(const f32x4*)(st + wide_read_row(q, c.lane) * kWideStride + col);
      if (!first)
        v[q] += __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, wide_elem_offset(vs, q, ld4), 0, kNT));
    }
#pragma unroll
    for (int q = 0; q < 16; ++q)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v[q]), rs, wide_elem_offset(vs, q, ld4), 0, kNT);
  }
};

// ---------------------------------------------------------------------------
// Block reductions (fixed order: deterministic)
// ---------------------------------------------------------------------------

template <int NT, class T, class Op>
__device__ __forceinline__ T block_reduce(T v, T* s_buf, Op op) {
  const int tid = threadIdx.x;
  s_buf[tid] = v;
  __syncthreads();
#pragma unroll
  for (int w = NT / 2; w > 0; w >>= 1) {
    if (tid < w) s_buf[tid] = op(s_buf[tid], s_buf[tid + w]);
    __syncthreads();
  }
  T r = s_buf[0];
  __syncthreads();
  return r;
}

struct OpMax { __device__ float operator()(float a, float b) const { return fmaxf(a, b); } };
struct OpAddF { __device__ float operator()(float a, float b) const { return a + b; } };
struct OpAddD { __device__ double operator()(double a, double b) const { return a + b; } };
struct OpAddI { __device__ int operator()(int a, int b) const { return a + b; } };

// Teacher distribution of one row: a_k = logit_k / tau kept in s_a, and the
// log normaliser log sum_k exp(a_k).  p_k = exp(a_k - lse_a).  Used by both
// the KL kernel and the teacher-probability kernel of the backward-only call,
// so that the loss and the gradient see the same p.
template <int NT>
__device__ __forceinline__ float teacher_row(const float* logit_row, int K, float inv_tau,
                                             float* s_a, float* s_red) {
  float mx = -INFINITY;
  for (int k = threadIdx.x; k < K; k += NT) {
    const float a = logit_row[k] * inv_tau;
    s_a[k] = a;
    mx = fmaxf(mx, a);
  }
  mx = block_reduce<NT>(mx, s_red, OpMax());
  float sm = 0.f;
  for (int k = threadIdx.x; k < K; k += NT) sm += expf(s_a[k] - mx);
  sm = block_reduce<NT>(sm, s_red, OpAddF());
  return mx + logf(sm);
}

// The sparse teacher target of one row for the recompute epilogue, with
// repeated ids merged: P[t, v] = sum of p_k over the k with idx[t, k] = v.
// The (id, k) pairs are sorted in LDS (bitonic, Kp keys, Kp a power of two
// >= K); the first k of each id receives P, summed over that id's entries in
// increasing k, and its later entries receive 0.  The epilogue subtracts
// every (t, k) entry of its hit lists, so each (t, v) loses exactly one
// nonzero term whatever order the lists hold, and the gradient is the same
// bit for bit from call to call.  With distinct ids psel[k] = p_k.  Ids
// outside [0, V) sort last and get no value (they have no hit-list entry).
__device__ __forceinline__ uint32_t key_k(unsigned long long key) { return (uint32_t)key; }
__device__ __forceinline__ uint32_t key_id(unsigned long long key) { return (uint32_t)(key >> 32); }

template <int NT>
__device__ __forceinline__ void merged_target_row(const int32_t* idx_row, int K, int Kp, int V, const float* s_a,
                                                  float lse_a, unsigned long long* s_key, float* psel_row) {
  constexpr unsigned long long kNone = ~0ull;
  // Rows rarely repeat an id: for K <= kDupScanK a pairwise scan (each id
  // against the ids before it, read four at a time from LDS) decides first,
  // and a row without repeats takes p_k as it is.  The outcome does not
  // depend on timing, and either path gives the same P.
  constexpr int kDupScanK = 512;
  __shared__ int s_dup;
  if (K <= kDupScanK) {
    int* s_id = (int*)s_key;                   // Kp >= K ints fit the key array
    for (int k = threadIdx.x; k < Kp; k += NT) s_id[k] = k < K ? idx_row[k] : -1;
    if (threadIdx.x == 0) s_dup = 0;
    __syncthreads();
    for (int k = threadIdx.x; k < K; k += NT) {
      const int id = s_id[k];
      if (id < 0 || id >= V) continue;
      bool dup = false;
      for (int k2 = 0; k2 < (k & ~3) && !dup; k2 += 4) {
        const int4 w = *(const int4*)(s_id + k2);
        dup = w.x == id || w.y == id || w.z == id || w.w == id;
      }
      for (int k2 = k & ~3; k2 < k && !dup; ++k2) dup = s_id[k2] == id;
      if (dup) s_dup = 1;
    }
    __syncthreads();
    const bool any = s_dup != 0;
    __syncthreads();                           // s_id is overwritten below
    if (!any) {
      for (int k = threadIdx.x; k < K; k += NT) {
        const int id = idx_row[k];
        if (id >= 0 && id < V) psel_row[k] = expf(s_a[k] - lse_a);
      }
      return;
    }
  }
  for (int k = threadIdx.x; k < Kp; k += NT) {
    unsigned long long key = kNone;
    if (k < K) {
      const int id = idx_row[k];
      if (id >= 0 && id < V) key = ((unsigned long long)(uint32_t)id << 32) | (uint32_t)k;
    }
    s_key[k] = key;
  }
  __syncthreads();
  for (int size = 2; size <= Kp; size <<= 1)
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < Kp / 2; i += NT) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool up = (lo & size) == 0;
        const unsigned long long a = s_key[lo], b = s_key[hi];
        if ((a > b) == up) {
          s_key[lo] = b;
          s_key[hi] = a;
        }
      }
      __syncthreads();
    }
  for (int i = threadIdx.x; i < K; i += NT) {
    const unsigned long long key = s_key[i];
    if (key == kNone) continue;
    const uint32_t id = key_id(key);
    if (i > 0 && key_id(s_key[i - 1]) == id) {
      psel_row[key_k(key)] = 0.f;
      continue;
    }
    float P = 0.f;
    for (int j = i; j < K && s_key[j] != kNone && key_id(s_key[j]) == id; ++j)
      P += expf(s_a[key_k(s_key[j])] - lse_a);
    psel_row[key_k(key)] = P;
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Small kernels
// ---------------------------------------------------------------------------

// N = number of counted positions; clears the loss accumulator and status.
__global__ __launch_bounds__(1024) void prep_kernel(const uint8_t* mask, int64_t T, int* count,
                                                    double* loss_acc, int32_t* status) {
  __shared__ int s_red[1024];
  int c = 0;
  for (int64_t t = threadIdx.x; t < T; t += 1024) c += mask ? (mask[t] != 0) : 1;
  c = block_reduce<1024>(c, s_red, OpAddI());
  if (threadIdx.x == 0) {
    *count = c;
    *loss_acc = 0.0;
    if (status) *status = 0;
  }
}

// Teacher-id hit lists of a chunk, filed by forward-GEMM wave tile: one
// block per 64-row group g of the chunk sorts the group's (t, k) entries by
// vocabulary strip id / kHitV (counting sort in LDS: count, scan, fill).
// Group g owns the fixed range [g 64 K, (g + 1) 64 K) of `hits`, so no
// global scan is needed; off[g (nvt + 1) + vt] is where strip vt's list
// starts, off[g (nvt + 1) + vt + 1] where it ends.  Entries of one list come
// in any order; each names its own output slot, so results do not depend on
// it.  Groups past the chunk's rows (up to the GEMM tiles' extent) get empty
// lists.  Dynamic LDS: nvt + 1 ints.
__global__ __launch_bounds__(1024) void hit_build_kernel(const int32_t* idx, int R, int K, int V, int nvt, int* off,
                                                         uint2* hits) {
  extern __shared__ int s_h[];
  __shared__ int s_w[16];
  const int g = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int t0 = g * kHitT;
  const int rows = max(0, min(kHitT, R - t0));
  const int n = rows * K;
  const int base = t0 * K;
  const int32_t* ids = idx + (int64_t)t0 * K;
  for (int i = tid; i <= nvt; i += 1024) s_h[i] = 0;
  __syncthreads();
  for (int e = tid; e < n; e += 1024) {
    const int id = ids[e];
    if (id >= 0 && id < V) atomicAdd(&s_h[id / kHitV], 1);
  }
  __syncthreads();
  // exclusive scan of s_h[0, nvt): contiguous pieces per thread, wave scan
  // of the piece sums, wave totals through LDS
  const int per = (nvt + 1023) / 1024;
  const int a = min(nvt, tid * per), b = min(nvt, a + per);
  int sum = 0;
  for (int i = a; i < b; ++i) sum += s_h[i];
  int incl = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == 63) s_w[w] = incl;
  __syncthreads();
  int run = incl - sum, total = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    run += i < w ? s_w[i] : 0;
    total += s_w[i];
  }
  for (int i = a; i < b; ++i) {
    const int c = s_h[i];
    s_h[i] = run;
    run += c;
  }
  __syncthreads();
  int* o = off + (int64_t)g * (nvt + 1);
  for (int i = tid; i < nvt; i += 1024) o[i] = base + s_h[i];
  if (tid == 0) o[nvt] = base + total;
  __syncthreads();
  for (int e = tid; e < n; e += 1024) {
    const int id = ids[e];
    if (id < 0 || id >= V) continue;
    const int pos = base + atomicAdd(&s_h[id / kHitV], 1);
    const int t = e / K;                             // row within the group
    hits[pos] = make_uint2((uint32_t)(base + e), hit_code(id, t));
  }
}

// dst[c][r] = src[r][c] for r < rows, c < cols; zero elsewhere in the
// [dst_rows x ld_dst] destination.  64x64 tiles through LDS.
template <class E>
__global__ __launch_bounds__(256) void transpose_pad_kernel(const typename E::T* src, int64_t ld_src,
                                                            int64_t rows, int64_t cols,
                                                            typename E::T* dst, int64_t ld_dst) {
  typedef typename E::T T;
  __shared__ T tile[64][65];
  const int64_t r0 = (int64_t)blockIdx.x * 64, c0 = (int64_t)blockIdx.y * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) {
    const int64_t r = r0 + i, c = c0 + tx;
    tile[i][tx] = (r < rows && c < cols) ? src[r * ld_src + c] : (T)0;
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int64_t c = c0 + i, r = r0 + tx;
    dst[c * ld_dst + r] = tile[tx][i];
  }
}

// bf16 transpose with 16-byte loads and stores: dst[c][r] = src[r][c] for
// r < rows, c < cols, zero elsewhere in the block's 64 x 64 destination
// tile.  Requires ld_src and ld_dst multiples of 8 and 16-byte aligned
// bases.
__global__ __launch_bounds__(256) void transpose_bf16_vec_kernel(const uint16_t* src, int64_t ld_src, int64_t rows,
                                                                 int64_t cols, uint16_t* dst, int64_t ld_dst) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[64][72];   // 144-byte rows
  const int64_t r0 = (int64_t)blockIdx.x * 64, c0 = (int64_t)blockIdx.y * 64;
  const int t = threadIdx.x;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int row = (t >> 3) + 32 * h, vc = t & 7;
    const int64_t r = r0 + row, c = c0 + 8 * vc;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r < rows) {
      if (c + 8 <= cols) {
        v = *(const u32x4*)(src + r * ld_src + c);
      } else if (c < cols) {
        uint16_t e8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) e8[e] = c + e < cols ? src[r * ld_src + c + e] : (uint16_t)0;
        v = u32x4{e8[0] | ((uint32_t)e8[1] << 16), e8[2] | ((uint32_t)e8[3] << 16), e8[4] | ((uint32_t)e8[5] << 16),
                  e8[6] | ((uint32_t)e8[7] << 16)};
      }
    }
    *(u32x4*)&tile[row][8 * vc] = v;
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int drow = (t >> 3) + 32 * h, vr = t & 7;
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = (uint32_t)tile[8 * vr + 2 * e][drow] | ((uint32_t)tile[8 * vr + 2 * e + 1][drow] << 16);
    *(u32x4*)(dst + (c0 + drow) * ld_dst + r0 + 8 * vr) = u32x4{w[0], w[1], w[2], w[3]};
  }
}

// dst[r][c] = src[r][c] for r < rows, c < cols; zero elsewhere in the
// [dst_rows x ld_dst] destination.
template <class E>
__global__ __launch_bounds__(256) void pad_kernel(const typename E::T* src, int64_t ld_src, int64_t rows,
                                                  int64_t cols, typename E::T* dst, int64_t ld_dst,
                                                  int64_t dst_rows) {
  typedef typename E::T T;
  const int64_t n = dst_rows * ld_dst;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / ld_dst, c = i - r * ld_dst;
    dst[i] = (r < rows && c < cols) ? src[r * ld_src + c] : (T)0;
  }
}


// Online logsumexp across vocabulary strips, first level: for each chunk row
// t and group of kMergeStrips strips, merge the per-strip (max, sum exp2)
// partials into one.  Block = 32 rows x 8 strip slices; consecutive threads
// read consecutive rows of one strip (coalesced); fixed merge order.  The
// second level (over the groups) is done by kl_rows_kernel.

__device__ __forceinline__ void lse_combine(float& M, float& L, float m2, float l2) {
  if (l2 <= 0.f) return;                      // empty: strip with no vocabulary rows
  if (m2 > M) { L = L * fast_exp2(M - m2) + l2; M = m2; }
  else L += l2 * fast_exp2(m2 - M);
}

__global__ __launch_bounds__(256) void lse_merge_kernel(const float2* part, int ldp, int nvt, int R, float2* part2) {
  __shared__ float s_m[8][32];
  __shared__ float s_l[8][32];
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  const int t = blockIdx.x * 32 + tx;
  const int v0 = blockIdx.y * kMergeStrips, v1 = min(nvt, v0 + kMergeStrips);
  float M = -INFINITY, L = 0.f;
  if (t < R) {
    for (int vt = v0 + ty; vt < v1; vt += 8) {
      const float2 p = part[(int64_t)vt * ldp + t];
      lse_combine(M, L, p.x, p.y);
    }
  }
  s_m[ty][tx] = M;
  s_l[ty][tx] = L;
  __syncthreads();
  if (ty == 0 && t < R) {
#pragma unroll
    for (int q = 1; q < 8; ++q) lse_combine(M, L, s_m[q][tx], s_l[q][tx]);
    part2[(int64_t)blockIdx.y * ldp + t] = make_float2(M, L);
  }
}

// One block per chunk row t:
//  1. the row's normaliser LSE_t from the ng group partials of lse_merge_kernel
//     (second level of the online logsumexp), written to lse2 / row_lse;
//  2. the teacher's distribution p over its K cached ids;
//  3. KL_t = sum_k p_k (log p_k - (z_k / tau - LSE_t)), with z_k the student
//     logit at id k captured by the forward epilogue.
// Invalid ids set *status and contribute nothing.
__global__ __launch_bounds__(256) void kl_rows_kernel(const float2* part2, int ldp, int ng, float* lse2_out,
                                                      float* row_lse, const float* zsel, const int32_t* idx,
                                                      const float* logit, int K, int V, float tau, double* rowkl,
                                                      float* row_kl, float* psel, int32_t* status) {
  extern __shared__ __attribute__((aligned(16))) char s_dyn[];   // teacher_lds_bytes(K)
  const int Kp = teacher_sort_len(K);
  unsigned long long* s_key = (unsigned long long*)s_dyn;
  float* s_a = (float*)(s_dyn + (size_t)Kp * 8);
  __shared__ float s_red[256];
  __shared__ double s_d[256];
  const int t = blockIdx.x, tid = threadIdx.x;

  // 1. LSE_t
  float M = -INFINITY, L = 0.f;
  for (int g = tid; g < ng; g += 256) {
    const float2 p = part2[(int64_t)g * ldp + t];
    lse_combine(M, L, p.x, p.y);
  }
  const float Mx = block_reduce<256>(M, s_red, OpMax());
  const float Ls = block_reduce<256>(L > 0.f ? L * fast_exp2(M - Mx) : 0.f, s_red, OpAddF());
  const float lse2 = Mx + __log2f(Ls);
  if (tid == 0) {
    lse2_out[t] = lse2;
    if (row_lse) row_lse[t] = lse2 * kLn2;
  }
  const float lse = lse2 * kLn2;              // natural-log normaliser of S = z / tau
  const float inv_tau = 1.f / tau;
  const float lse_a = teacher_row<256>(logit + (int64_t)t * K, K, inv_tau, s_a, s_red);
  double kl = 0.0;
  for (int k = tid; k < K; k += 256) {
    const int id = idx[(int64_t)t * K + k];
    if (id < 0 || id >= V) {
      if (status) *status = 7;                // KD_ERR_BAD_INDEX
      continue;
    }
    const float z = zsel[(int64_t)t * K + k];
    const float logp = s_a[k] - lse_a;
    const float p = expf(logp);
    if (p > 0.f) kl += (double)p * ((double)logp - ((double)z * inv_tau - (double)lse));
  }
  kl = block_reduce<256>(kl, s_d, OpAddD());
  // the recompute epilogue's sparse part, repeated ids merged
  if (psel) merged_target_row<256>(idx + (int64_t)t * K, K, Kp, V, s_a, lse_a, s_key, psel + (int64_t)t * K);
  if (tid == 0) {
    rowkl[t] = kl;
    if (row_kl) row_kl[t] = (float)kl;
  }
}

// loss_acc += sum_t m_t KL_t over the chunk, fixed order, fp64.
__global__ __launch_bounds__(256) void chunk_loss_kernel(const double* rowkl, const uint8_t* mask, int R,
                                                         double* loss_acc) {
  __shared__ double s_d[256];
  double s = 0.0;
  for (int t = threadIdx.x; t < R; t += 256)
    if (!mask || mask[t]) s += rowkl[t];
  s = block_reduce<256>(s, s_d, OpAddD());
  if (threadIdx.x == 0) *loss_acc += s;
}

// The sparse teacher target of the chunk's rows for the recompute epilogue,
// in the backward-only call (the fused call gets it from kl_rows_kernel):
// p_k with repeated ids merged (merged_target_row).  One block per chunk row;
// invalid ids set *status and are left out of the hit lists, so they
// contribute nothing.  Dynamic LDS: teacher_lds_bytes(K).
__global__ __launch_bounds__(128) void teacher_p_kernel(const int32_t* idx, const float* logit, int K, int V,
                                                        float tau, float* psel, int32_t* status) {
  extern __shared__ __attribute__((aligned(16))) char s_dyn[];
  const int Kp = teacher_sort_len(K);
  unsigned long long* s_key = (unsigned long long*)s_dyn;
  float* s_a = (float*)(s_dyn + (size_t)Kp * 8);
  __shared__ float s_red[128];
  const int t = blockIdx.x;
  const float lse_a = teacher_row<128>(logit + (int64_t)t * K, K, 1.f / tau, s_a, s_red);
  for (int k = threadIdx.x; k < K; k += 128) {
    const int id = idx[(int64_t)t * K + k];
    if ((id < 0 || id >= V) && status) *status = 7;   // KD_ERR_BAD_INDEX
  }
  merged_target_row<128>(idx + (int64_t)t * K, K, Kp, V, s_a, lse_a, s_key, psel + (int64_t)t * K);
}

// grad_hidden rows of the chunk: fixed-order sum of the split-K partials,
// stored as fp32 or (OutT = uint16_t) bf16 with round to nearest even.
__device__ __forceinline__ void store_out(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_out(uint16_t* p, float v) { *p = f32_to_bf16(v); }

template <class OutT>
__global__ __launch_bounds__(256) void dh_reduce_kernel(const float* part, int64_t ldp, int64_t split_stride,
                                                        int splits, int R, int d, OutT* out, int64_t ldo) {
  const int64_t n = (int64_t)R * d;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t t = i / d, j = i - t * d;
    const float* p = part + t * ldp + j;
    float s = 0.f;
    for (int sp = 0; sp < splits; ++sp) s += p[(int64_t)sp * split_stride];
    store_out(out + t * ldo + j, s);
  }
}

// The same with 4 columns per thread (d, ldp and ldo multiples of 4, the
// partial buffer and the output 16-byte / 8-byte aligned): one 16-byte load
// per split, same fixed summation order.
__device__ __forceinline__ void store_out4(float* p, float4 v) { *(float4*)p = v; }
__device__ __forceinline__ void store_out4(uint16_t* p, float4 v) {
  *(uint2*)p = make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
}

template <class OutT>
__global__ __launch_bounds__(256) void dh_reduce4_kernel(const float* part, int64_t ldp, int64_t split_stride,
                                                         int splits, int R, int d, OutT* out, int64_t ldo) {
  const int d4 = d >> 2;
  const int64_t n = (int64_t)R * d4;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t t = i / d4, j = 4 * (i - t * d4);
    const float* p = part + t * ldp + j;
    float4 s = *(const float4*)p;
    for (int sp = 1; sp < splits; ++sp) {
      const float4 v = *(const float4*)(p + (int64_t)sp * split_stride);
      s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
    store_out4(out + t * ldo + j, s);
  }
}

// bf16 copy (round to nearest even) of an fp32 array.
__global__ __launch_bounds__(256) void to_bf16_kernel(const float* src, uint16_t* dst, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    dst[i] = f32_to_bf16(src[i]);
}

__global__ void finalize_kernel(const double* loss_acc, const int* count, float tau, float* loss) {
  const int N = *count;
  *loss = N > 0 ? (float)((double)tau * (double)tau * (*loss_acc) / (double)N) : 0.f;
}

}  // namespace kd
