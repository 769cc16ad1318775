// kd_topk_kl.hip -- host side of the fused chunked top-K KL loss: argument
// checks, workspace carve-up and the per-chunk launch sequence, behind the C
// ABI declared in include/kd_topk_kl.h.
//
// Per call:
//   prep            N = #counted positions; clear the loss accumulator
//   transpose W     W^T (zero-padded) for the hidden-gradient GEMM
//   for each chunk of `chunk` rows (the method: only one chunk's logits
//   exist at any time; they are reduced into the loss, dropped, and formed
//   again for the gradient -- Glonce, "Multiverse Computing cuts LLM
//   distillation VRAM by 15x with chunked KL loss", paragraph on Multiverse's
//   two-part fix):
//     transpose H_c   H_c^T for the head-gradient GEMM; teacher-id hit lists
//     GEMM + LSE      z^T = W H_c^T, per-strip (max, sum exp) partials, and
//                     z at the teacher ids picked from the accumulators
//     KL rows         online merge -> LSE_t; teacher p; KL_t
//     chunk loss      fixed-order fp64 sum of m_t KL_t
//     GEMM + grad     recompute z^T, G = (tau/N) m (q - P) in two layouts,
//                     the sparse teacher part P at the hit lists' entries
//   (the backward-only entry point first recomputes the teacher's P)
//     GEMM dH         split-K over the vocabulary, fixed-order reduction
//     GEMM dW         grad_W (+)= G^T H in fp32, once per group of
//                     consecutive chunks spanning up to 8192 rows (their
//                     G^T and H^T sit side by side in the workspace)
//   finalize        loss = tau^2 * acc / N
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "../../include/kd_topk_kl.h"
#include "kd_cache.hpp"
#include "kd_plan.hpp"
#include "kd_kernels.hpp"
#include "kd_probe.hpp"

namespace kd {
namespace {

// (tile configurations, the plan and the workspace carve-up: kd_plan.hpp)

// One block per tile (a multiple of 8 blocks).
template <class TC, class E, class Epi>
hipError_t launch_gemm(const GemmShape& g, const Epi& epi, hipStream_t st) {
  const int nb = g.tiles_m * g.tiles_n * g.splits;
  const int grid = (nb + 7) & ~7;
  hipLaunchKernelGGL((gemm_nt_kernel<E, TC::BM, TC::BN, TC::WM, TC::WN, TC::STAGES, Epi, TC::RB>), dim3(grid),
                     dim3(TC::kThreads), 0, st, g, epi);
  return hipGetLastError();
}

// group_m: row tiles per group of the tile order (see tile_position).  The
// head-gradient GEMM uses 4 (it re-streams its 11.8 MB H_c^T operand once
// per row band otherwise); the others measured best with 1.
template <class TC>
GemmShape make_shape(const void* A, int64_t lda, int M, const void* B, int64_t ldb, int N, int64_t k_bytes,
                     int splits, int group_m) {
  GemmShape g;
  g.group_m = group_m;
  g.A = A; g.B = B; g.lda = lda; g.ldb = ldb; g.M = M; g.N = N;
  g.k_tiles = (int)(k_bytes / TC::RB);
  g.k_tiles_per_split = (int)cdiv(g.k_tiles, splits);
  g.splits = (int)cdiv(g.k_tiles, g.k_tiles_per_split);   // <= splits; no split is empty
  g.tiles_m = (int)cdiv(M, TC::BM);
  g.tiles_n = (int)cdiv(N, TC::BN);
  return g;
}

// dst [gy*64 x ld_dst] = transpose of src [rows x cols] (ld_src), zero
// padded; 16-byte accesses when the layout allows it.
template <class E>
void launch_transpose(const typename E::T* src, int64_t ld_src, int64_t rows, int64_t cols, typename E::T* dst,
                      int64_t ld_dst, unsigned gx, unsigned gy, hipStream_t st) {
  const bool vec = E::kBytes == 2 && ld_src % 8 == 0 && ld_dst % 8 == 0 &&
                   ((((uintptr_t)src) | ((uintptr_t)dst)) & 15) == 0;
  if (vec)
    hipLaunchKernelGGL(transpose_bf16_vec_kernel, dim3(gx, gy), dim3(256), 0, st, (const uint16_t*)src, ld_src, rows,
                       cols, (uint16_t*)dst, ld_dst);
  else
    hipLaunchKernelGGL(transpose_pad_kernel<E>, dim3(gx, gy), dim3(256), 0, st, src, ld_src, rows, cols, dst, ld_dst);
}

#define KD_LAUNCH_CHECK()                         \
  do {                                            \
    if (hipGetLastError() != hipSuccess) return KD_ERR_HIP; \
  } while (0)

// Pointers of one call (see the entry points for which a mode uses).
struct Args {
  const void* hidden;
  const void* W;
  const int32_t* idx;
  const float* logit;
  const uint8_t* mask;
  float tau;
  float* loss;             // fused, forward
  float* row_lse;          // fused, forward: output (may be NULL in fused); backward: input
  float* row_kl;           // fused, forward: output or NULL
  const float* grad_loss;  // backward: device scalar dL/dloss, or NULL for 1
  void* grad_hidden;       // fused, backward (NULL in backward: not computed)
  int32_t gh_dtype;        // KD_F32 or KD_BF16
  float* grad_W;           // fused, backward (NULL in backward: not computed)
  int accumulate_W;        // backward: add into grad_W instead of overwriting it
  uint16_t* grad_W_bf16;   // backward: optional bf16 copy of the final grad_W
  int32_t* status;
  hipStream_t st;
  void* const* events;     // fused timing markers or NULL
};

template <class E>
int32_t run(const Plan& P, const Args& A, char* ws) {
  typedef typename E::T T;
  hipStream_t st = A.st;
  // timing markers (measurement entry point only)
  auto mark = [&](int64_t slot, int end) {
    if (A.events) (void)hipEventRecord((hipEvent_t)A.events[2 * slot + end], st);
  };
  // a phase this call does not run: both markers back to back (every event
  // is recorded in every call, so each phase reads as a valid interval)
  auto skip = [&](int64_t slot) {
    mark(slot, 0);
    mark(slot, 1);
  };
  const int64_t pro_slot = (int64_t)KD_NUM_PHASES * P.nchunks;
  int* count = (int*)(ws + P.off_scalar);
  double* loss_acc = (double*)(ws + P.off_scalar + 8);
  T* Wt = (T*)(ws + P.off_wt);
  T* Wp = (T*)(ws + P.off_wp);
  T* Hp = (T*)(ws + P.off_hp);
  T* Ht = (T*)(ws + P.off_ht);
  T* G = (T*)(ws + P.off_g);
  T* Gt = (T*)(ws + P.off_gt);
  float2* part = (float2*)(ws + P.off_part);
  float* lse2 = (float*)(ws + P.off_lse2);
  double* rowkl = (double*)(ws + P.off_rowkl);
  float* dhp = (float*)(ws + P.off_dh);
  int* hoff = (int*)(ws + P.off_hoff);
  uint2* hits = (uint2*)(ws + P.off_hits);
  float* zsel = (float*)(ws + P.off_zsel);
  float2* part2 = (float2*)(ws + P.off_part2);
  float* psel = P.bwd ? (float*)(ws + P.off_psel) : nullptr;

  const int64_t T_ = P.T, d = P.d, V = P.V, K = P.K;
  const float tau = A.tau;
  const float c2 = kLog2e / tau;
  const bool want_dh = P.bwd && A.grad_hidden, want_dw = P.bwd && A.grad_W;

  mark(pro_slot, 0);
  hipLaunchKernelGGL(prep_kernel, dim3(1), dim3(1024), 0, st, A.mask, T_, count, loss_acc, A.status);
  KD_LAUNCH_CHECK();
  if (want_dh) {
    // W^T, zero-padded to [d_p][V_p]
    launch_transpose<E>((const T*)A.W, d, V, d, Wt, P.V_p, (unsigned)(P.V_p / 64), (unsigned)(P.d_p / 64), st);
    KD_LAUNCH_CHECK();
  }
  const T* Wsrc = (const T*)A.W;
  int64_t ldw = d;
  if (P.pad_d) {
    const int64_t n = V * P.d_p;
    hipLaunchKernelGGL(pad_kernel<E>, dim3((unsigned)std::min<int64_t>(cdiv(n, 256), 65536)), dim3(256), 0, st,
                       (const T*)A.W, d, V, d, Wp, P.d_p, V);
    KD_LAUNCH_CHECK();
    Wsrc = Wp;
    ldw = P.d_p;
  }
  const int64_t kbytes_d = P.d_p * P.eb;
  mark(pro_slot, 1);

  for (int64_t c = 0; c < P.nchunks; ++c) {
    const int64_t c0 = c * P.chunk;
    const int R = (int)std::min<int64_t>(P.chunk, T_ - c0);
    const int64_t Rt = round_up(R, kBN);     // rows covered by the GEMM tiles this chunk
    const int64_t slot = c * KD_NUM_PHASES;
    // the chunk's column slot in G^T / H_c^T; the head-gradient GEMM runs
    // once per group of dw_group chunks, over all of the group's rows
    const int64_t gslot = c % P.dw_group;
    const bool group_end = gslot == P.dw_group - 1 || c == P.nchunks - 1;
    const uint8_t* mask_c = A.mask ? A.mask + c0 : nullptr;
    const int32_t* idx_c = A.idx + c0 * K;
    const float* logit_c = A.logit + c0 * K;
    mark(slot + 0, 0);
    const T* Hc = (const T*)A.hidden + c0 * d;
    const T* Hsrc = Hc;
    int64_t ldh = d;
    if (P.pad_d) {
      const int64_t n = Rt * P.d_p;
      hipLaunchKernelGGL(pad_kernel<E>, dim3((unsigned)std::min<int64_t>(cdiv(n, 256), 65536)), dim3(256), 0, st,
                         Hc, d, (int64_t)R, d, Hp, P.d_p, Rt);
      KD_LAUNCH_CHECK();
      Hsrc = Hp;
      ldh = P.d_p;
    }
    if (want_dw) {
      // H_c^T, zero-padded to [d_p][R_p], into the chunk's slot of the group
      launch_transpose<E>(Hc, d, (int64_t)R, d, Ht + gslot * P.R_p, P.R_g, (unsigned)(P.R_p / 64),
                          (unsigned)(P.d_p / 64), st);
      KD_LAUNCH_CHECK();
    }
    // teacher-id hit lists for the forward and the recompute epilogues
    hipLaunchKernelGGL(hit_build_kernel, dim3((unsigned)(Rt / kHitT)), dim3(1024),
                       (size_t)(P.nvt + 1) * sizeof(int), st, idx_c, R, (int)K, (int)V, (int)P.nvt, hoff, hits);
    KD_LAUNCH_CHECK();
    mark(slot + 0, 1);

    if (P.fwd) {
      // forward: z^T = W H_c^T -> LSE partials, z at the teacher ids
      mark(slot + 1, 0);
      {
        GemmShape g = make_shape<TileMain>(Wsrc, ldw, (int)V, Hsrc, ldh, R, kbytes_d, 1, 1);
        EpiLsePartial epi{part, (int)P.R_p, (int)V, c2, hoff, hits, zsel, (int)(P.nvt + 1)};
        if (launch_gemm<TileMain, E>(g, epi, st) != hipSuccess) return KD_ERR_HIP;
      }
      mark(slot + 1, 1);
      mark(slot + 2, 0);
      hipLaunchKernelGGL(lse_merge_kernel, dim3((unsigned)cdiv(R, 32), (unsigned)P.ng), dim3(256), 0, st,
                         (const float2*)part, (int)P.R_p, (int)P.nvt, R, part2);
      KD_LAUNCH_CHECK();
      hipLaunchKernelGGL(kl_rows_kernel, dim3(R), dim3(256), teacher_lds_bytes((int)K), st, (const float2*)part2,
                         (int)P.R_p, (int)P.ng,
                         lse2, A.row_lse ? A.row_lse + c0 : nullptr, (const float*)zsel, idx_c, logit_c, (int)K,
                         (int)V, tau, rowkl, A.row_kl ? A.row_kl + c0 : nullptr, psel, A.status);
      KD_LAUNCH_CHECK();
      hipLaunchKernelGGL(chunk_loss_kernel, dim3(1), dim3(256), 0, st, (const double*)rowkl, mask_c, R, loss_acc);
      KD_LAUNCH_CHECK();
      mark(slot + 2, 1);
    } else {
      skip(slot + 1);
      skip(slot + 2);
    }
    if (!P.bwd) {
      for (int p = 3; p < KD_NUM_PHASES; ++p) skip(slot + p);
      continue;
    }
    // backward-only call: the teacher probabilities the forward's KL kernel
    // would have left (phase 4, recorded ahead of phase 3)
    mark(slot + 4, 0);
    if (!P.fwd) {
      hipLaunchKernelGGL(teacher_p_kernel, dim3(R), dim3(128), teacher_lds_bytes((int)K), st, idx_c, logit_c,
                         (int)K, (int)V, tau, psel, A.status);
      KD_LAUNCH_CHECK();
    }
    mark(slot + 4, 1);

    mark(slot + 3, 0);
    // backward recompute: G = (tau/N) m q, both layouts; the row normaliser
    // comes from this call's forward (base 2) or from the saved row_lse
    // (natural log)
    {
      const float* lse_src = P.fwd ? (const float*)lse2 : (const float*)A.row_lse + c0;
      const float lse_to2 = P.fwd ? 1.f : kLog2e;
      GemmShape g = make_shape<TileMain>(Wsrc, ldw, (int)V, Hsrc, ldh, R, kbytes_d, 1, 1);
      // the sparse teacher part goes in the epilogue, through the hit lists
      EpiGrad<E> epi{G, P.V_p, Gt + gslot * P.R_p, P.R_g, lse_src, lse_to2, mask_c, count, A.grad_loss, tau, c2,
                     (int)V, R, hoff, hits, psel, (int)(P.nvt + 1)};
      if (launch_gemm<TileMain, E>(g, epi, st) != hipSuccess) return KD_ERR_HIP;
    }
    mark(slot + 3, 1);
    if (want_dh) {
      mark(slot + 5, 0);
      // dH_c = G W  (A = G [Rt x V_p], B = W^T [d x V_p]), split-K over V
      EpiStoreSplit epi{dhp, P.Nd_p, P.R_p * P.Nd_p};
      GemmShape g;
      if (P.dh_bn == TileDhWide::BN) {
        g = make_shape<TileDhWide>(G, P.V_p, R, Wt, P.V_p, (int)d, P.V_p * P.eb, P.splits, 8);
        if (launch_gemm<TileDhWide, E>(g, epi, st) != hipSuccess) return KD_ERR_HIP;
      } else {
        g = make_shape<TileMain>(G, P.V_p, R, Wt, P.V_p, (int)d, P.V_p * P.eb, P.splits, 8);
        if (launch_gemm<TileMain, E>(g, epi, st) != hipSuccess) return KD_ERR_HIP;
      }
      mark(slot + 5, 1);
      mark(slot + 6, 0);
      const int64_t n = (int64_t)R * d;
      const dim3 grid((unsigned)std::min<int64_t>(cdiv(n, 256), 65536));
      const bool v4 = d % 4 == 0;
      const dim3 grid4((unsigned)std::min<int64_t>(cdiv(n / 4, 256), 65536));
      if (A.gh_dtype == KD_BF16) {
        uint16_t* o = (uint16_t*)A.grad_hidden + c0 * d;
        if (v4)
          hipLaunchKernelGGL(dh_reduce4_kernel<uint16_t>, grid4, dim3(256), 0, st, (const float*)dhp, P.Nd_p,
                             P.R_p * P.Nd_p, g.splits, R, (int)d, o, d);
        else
          hipLaunchKernelGGL(dh_reduce_kernel<uint16_t>, grid, dim3(256), 0, st, (const float*)dhp, P.Nd_p,
                             P.R_p * P.Nd_p, g.splits, R, (int)d, o, d);
      } else {
        float* o = (float*)A.grad_hidden + c0 * d;
        if (v4)
          hipLaunchKernelGGL(dh_reduce4_kernel<float>, grid4, dim3(256), 0, st, (const float*)dhp, P.Nd_p,
                             P.R_p * P.Nd_p, g.splits, R, (int)d, o, d);
        else
          hipLaunchKernelGGL(dh_reduce_kernel<float>, grid, dim3(256), 0, st, (const float*)dhp, P.Nd_p,
                             P.R_p * P.Nd_p, g.splits, R, (int)d, o, d);
      }
      KD_LAUNCH_CHECK();
      mark(slot + 6, 1);
    } else {
      skip(slot + 5);
      skip(slot + 6);
    }
    if (want_dw) {
      mark(slot + 7, 0);
      if (group_end) {
        // dW (+)= G^T H^T over the group's rows (A = G^T [V_p x R_g], B =
        // H^T [d x R_g]); a slot's columns past its chunk's rows are zero
        // in H^T, and the last slot is contracted up to its tile rows
        const int64_t kbytes = (gslot * P.R_p + Rt) * P.eb;
        EpiAccum epi{A.grad_W, d, (int)V, (int)d, (c == gslot && !A.accumulate_W) ? 1 : 0};
        if (P.dw_wide && (((uintptr_t)A.grad_W) & 15) == 0) {
          GemmShape g = make_shape<TileDhWide>(Gt, P.R_g, (int)V, Ht, P.R_g, (int)d, kbytes, 1, 4);
          if (launch_gemm<TileDhWide, E>(g, epi, st) != hipSuccess) return KD_ERR_HIP;
        } else if (P.dw_bn == TileHead::BN) {
          GemmShape g = make_shape<TileHead>(Gt, P.R_g, (int)V, Ht, P.R_g, (int)d, kbytes, 1, 4);
          if (launch_gemm<TileHead, E>(g, epi, st) != hipSuccess) return KD_ERR_HIP;
        } else {
          GemmShape g = make_shape<TileHeadNarrow>(Gt, P.R_g, (int)V, Ht, P.R_g, (int)d, kbytes, 1, 4);
          if (launch_gemm<TileHeadNarrow, E>(g, epi, st) != hipSuccess) return KD_ERR_HIP;
        }
      }
      mark(slot + 7, 1);
    } else {
      skip(slot + 7);
    }
  }
  mark(pro_slot + 1, 0);
  if (P.fwd) {
    hipLaunchKernelGGL(finalize_kernel, dim3(1), dim3(1), 0, st, (const double*)loss_acc, (const int*)count, tau,
                       A.loss);
    KD_LAUNCH_CHECK();
  }
  if (want_dw && A.grad_W_bf16) {
    const int64_t n = V * d;
    hipLaunchKernelGGL(to_bf16_kernel, dim3((unsigned)std::min<int64_t>(cdiv(n, 256), 65536)), dim3(256), 0, st,
                       (const float*)A.grad_W, A.grad_W_bf16, n);
    KD_LAUNCH_CHECK();
  }
  mark(pro_slot + 1, 1);
  return KD_OK;
}

int32_t dispatch(int mode, int32_t in_dtype, int64_t T, int64_t d, int64_t V, int64_t K, int64_t chunk,
                 void* workspace, size_t workspace_bytes, const Args& A, bool lean = false) {
  if (!(A.tau > 0.f) || !isfinite(A.tau)) return KD_ERR_BAD_TAU;
  Plan p;
  const int32_t st = make_plan(T, d, V, K, chunk, in_dtype, mode, &p, lean);
  if (st != KD_OK) return st;
  if ((((uintptr_t)A.hidden) | ((uintptr_t)A.W)) & 15) return KD_ERR_BAD_SHAPE;
  if (lean && p.total > workspace_bytes) return KD_ERR_NOALLOC_SIZE;
  if (!workspace || workspace_bytes < p.total || (((uintptr_t)workspace) & 255)) return KD_ERR_WORKSPACE;
  if (in_dtype == KD_BF16) return run<Bf16>(p, A, (char*)workspace);
  return run<F32>(p, A, (char*)workspace);
}

// ---------------------------------------------------------------------------
// Fixed device scratch of the allocation-free entry point: a file-scope
// device array that each GPU the library runs on holds from the library's
// first use on it until the process ends.  Host code never passes the
// array's name to a kernel or a copy (on the host it names a stand-in, not
// device memory): the device address is looked up once per device with
// hipGetSymbolAddress, with that device current, and kept.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[KD_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the device that `stream` belongs to (the
// current device for the null stream).
int32_t scratch_address(hipStream_t stream, void** out) {
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return KD_ERR_HIP;
  int dev = cur;
  if (stream) {
    hipDevice_t sd;
    if (hipStreamGetDevice(stream, &sd) != hipSuccess) return KD_ERR_HIP;
    dev = (int)sd;
  }
  if (dev < 0 || dev >= kMaxDevices) return KD_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return KD_ERR_HIP;
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (dev != cur) (void)hipSetDevice(cur);
    if (e != hipSuccess || !ptr) return KD_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return KD_OK;
}


// (the cache builder's plan: kd_plan.hpp)

template <class E>
int32_t run_cache(const CachePlan& P, const void* hidden, const void* W, int32_t* out_idx, float* out_logit, char* ws,
                  hipStream_t st, void* const* events) {
  typedef typename E::T T;
  // timing markers (measurement entry point only): slot c * KD_CACHE_PHASES + p
  // per chunk phase, slot KD_CACHE_PHASES * nchunks for the prologue
  auto mark = [&](int64_t slot, int end) {
    if (events) (void)hipEventRecord((hipEvent_t)events[2 * slot + end], st);
  };
  T* Wp = (T*)(ws + P.off_wp);
  T* Hp = (T*)(ws + P.off_hp);
  float* bmax = (float*)(ws + P.off_bmax);
  float* theta = (float*)(ws + P.off_theta);
  int* cnt = (int*)(ws + P.off_cnt);
  uint2* cand = (uint2*)(ws + P.off_cand);
  int* ovf = (int*)(ws + P.off_ovf);
  float* zc = (float*)(ws + P.off_z);
  const int64_t d = P.d, V = P.V, K = P.K;

  const T* Wsrc = (const T*)W;
  int64_t ldw = d;
  mark(KD_CACHE_PHASES * P.nchunks, 0);
  if (P.pad_d) {
    const int64_t n = V * P.d_p;
    hipLaunchKernelGGL(pad_kernel<E>, dim3((unsigned)std::min<int64_t>(cdiv(n, 256), 65536)), dim3(256), 0, st,
                       (const T*)W, d, V, d, Wp, P.d_p, V);
    KD_LAUNCH_CHECK();
    Wsrc = Wp;
    ldw = P.d_p;
  }
  mark(KD_CACHE_PHASES * P.nchunks, 1);
  const int64_t kbytes_d = P.d_p * P.eb;
  for (int64_t c = 0; c < P.nchunks; ++c) {
    const int64_t c0 = c * P.chunk;
    const int R = (int)std::min<int64_t>(P.chunk, P.T - c0);
    const int64_t slot = c * KD_CACHE_PHASES;
    mark(slot + 0, 0);
    const T* Hc = (const T*)hidden + c0 * d;
    const T* Hsrc = Hc;
    int64_t ldh = d;
    if (P.pad_d) {
      const int64_t Rt = round_up(R, kBN);
      const int64_t n = Rt * P.d_p;
      hipLaunchKernelGGL(pad_kernel<E>, dim3((unsigned)std::min<int64_t>(cdiv(n, 256), 65536)), dim3(256), 0, st,
                         Hc, d, (int64_t)R, d, Hp, P.d_p, Rt);
      KD_LAUNCH_CHECK();
      Hsrc = Hp;
      ldh = P.d_p;
    }
    GemmShape g = make_shape<TileMain>(Wsrc, ldw, (int)V, Hsrc, ldh, R, kbytes_d, 1, 1);
    if (launch_gemm<TileMain, E>(g, EpiBlockMax{bmax, (int)(P.V_p / kBlockRows), (int)V, zc, P.V_p}, st) !=
        hipSuccess)
      return KD_ERR_HIP;
    mark(slot + 0, 1);
    mark(slot + 1, 0);
    hipLaunchKernelGGL(cache_threshold_kernel, dim3(R), dim3(256), 0, st, (const float*)bmax,
                       (int)(P.V_p / kBlockRows), (int)P.nb32, (int)K, theta);
    KD_LAUNCH_CHECK();
    mark(slot + 1, 1);
    mark(slot + 2, 0);
    hipLaunchKernelGGL(cache_collect_kernel, dim3(R), dim3(256), 0, st, (const float*)zc, P.V_p, (int)V,
                       (const float*)theta, cnt, cand, P.cap);
    KD_LAUNCH_CHECK();
    mark(slot + 2, 1);
    mark(slot + 3, 0);
    int32_t* oi = out_idx + c0 * K;
    float* ol = out_logit + c0 * K;
    hipLaunchKernelGGL(cache_select_kernel, dim3(R), dim3(256), (size_t)P.cap * sizeof(uint64_t), st,
                       (const int*)cnt, (const uint2*)cand, P.cap, (int)K, oi, ol, ovf);
    KD_LAUNCH_CHECK();
    hipLaunchKernelGGL(cache_fallback_kernel<E>, dim3(R), dim3(256), (size_t)2 * P.half * sizeof(uint64_t), st, Hc,
                       d, (const T*)W, d, (int)d, (int)V, (int)K, P.half, (const int*)ovf, oi, ol);
    KD_LAUNCH_CHECK();
    mark(slot + 3, 1);
  }
  return KD_OK;
}

}  // namespace
}  // namespace kd

extern "C" {

size_t kd_topk_kl_workspace_bytes(int64_t T, int64_t d, int64_t V, int64_t K, int64_t chunk, int32_t in_dtype) {
  return kd::workspace_for(kd::kFused, T, d, V, K, chunk, in_dtype);
}

size_t kd_topk_kl_fwd_workspace_bytes(int64_t T, int64_t d, int64_t V, int64_t K, int64_t chunk, int32_t in_dtype) {
  return kd::workspace_for(kd::kForward, T, d, V, K, chunk, in_dtype);
}

size_t kd_topk_kl_bwd_workspace_bytes(int64_t T, int64_t d, int64_t V, int64_t K, int64_t chunk, int32_t in_dtype) {
  return kd::workspace_for(kd::kBackward, T, d, V, K, chunk, in_dtype);
}

int32_t kd_topk_kl_dw_chunks(int64_t T, int64_t d, int64_t V, int64_t K, int64_t chunk, int32_t in_dtype) {
  kd::Plan p;
  if (kd::make_plan(T, d, V, K, chunk, in_dtype, kd::kFused, &p) != KD_OK) return 0;
  return p.dw_group;
}

static int32_t fwd_bwd_impl(const void* hidden, const void* W, int32_t in_dtype, const int32_t* teacher_idx,
                            const float* teacher_logit, const uint8_t* mask, int64_t T, int64_t d, int64_t V,
                            int64_t K, float tau, int64_t chunk, float* loss, float* grad_hidden, float* grad_W,
                            float* row_lse, float* row_kl, void* workspace, size_t workspace_bytes,
                            int32_t* status_dev, void* stream, void* const* events) {
  if (!hidden || !W || !teacher_idx || !teacher_logit || !loss || !grad_hidden || !grad_W) return KD_ERR_NULL_ARG;
  kd::Args a{hidden, W, teacher_idx, teacher_logit, mask, tau, loss, row_lse, row_kl, nullptr, grad_hidden, KD_F32,
             grad_W, 0, nullptr, status_dev, (hipStream_t)stream, events};
  return kd::dispatch(kd::kFused, in_dtype, T, d, V, K, chunk, workspace, workspace_bytes, a);
}

int32_t kd_topk_kl_fwd_bwd(const void* hidden, const void* W, int32_t in_dtype, const int32_t* teacher_idx,
                           const float* teacher_logit, const uint8_t* mask, int64_t T, int64_t d, int64_t V,
                           int64_t K, float tau, int64_t chunk, float* loss, float* grad_hidden, float* grad_W,
                           float* row_lse, float* row_kl, void* workspace, size_t workspace_bytes,
                           int32_t* status_dev, void* stream) {
  return fwd_bwd_impl(hidden, W, in_dtype, teacher_idx, teacher_logit, mask, T, d, V, K, tau, chunk, loss,
                      grad_hidden, grad_W, row_lse, row_kl, workspace, workspace_bytes, status_dev, stream, nullptr);
}

int32_t kd_topk_kl_fwd_bwd_noalloc(const void* hidden, const void* W, int32_t in_dtype, const int32_t* teacher_idx,
                                   const float* teacher_logit, const uint8_t* mask, int64_t T, int64_t d, int64_t V,
                                   int64_t K, float tau, int64_t chunk, float* loss, float* grad_hidden,
                                   float* grad_W, float* row_lse, float* row_kl, int32_t* status_dev,
                                   void* stream) {
  if (!hidden || !W || !teacher_idx || !teacher_logit || !loss || !grad_hidden || !grad_W) return KD_ERR_NULL_ARG;
  kd::Args a{hidden, W, teacher_idx, teacher_logit, mask, tau, loss, row_lse, row_kl, nullptr, grad_hidden, KD_F32,
             grad_W, 0, nullptr, status_dev, (hipStream_t)stream, nullptr};
  // argument and size checks come first, so a call that cannot run touches
  // no device state
  kd::Plan p;
  const int32_t st = kd::make_plan(T, d, V, K, chunk, in_dtype, kd::kFused, &p, true);
  if (st != KD_OK) return st;
  if (!(tau > 0.f) || !isfinite(tau)) return KD_ERR_BAD_TAU;
  if (p.total > KD_NOALLOC_SCRATCH_BYTES) return KD_ERR_NOALLOC_SIZE;
  void* ws = nullptr;
  const int32_t se = kd::scratch_address((hipStream_t)stream, &ws);
  if (se != KD_OK) return se;
  return kd::dispatch(kd::kFused, in_dtype, T, d, V, K, chunk, ws, KD_NOALLOC_SCRATCH_BYTES, a, true);
}

int32_t kd_topk_kl_fwd_bwd_timed(const void* hidden, const void* W, int32_t in_dtype, const int32_t* teacher_idx,
                                 const float* teacher_logit, const uint8_t* mask, int64_t T, int64_t d, int64_t V,
                                 int64_t K, float tau, int64_t chunk, float* loss, float* grad_hidden, float* grad_W,
                                 float* row_lse, float* row_kl, void* workspace, size_t workspace_bytes,
                                 int32_t* status_dev, void* stream, void* const* events) {
  if (!events) return KD_ERR_NULL_ARG;
  return fwd_bwd_impl(hidden, W, in_dtype, teacher_idx, teacher_logit, mask, T, d, V, K, tau, chunk, loss,
                      grad_hidden, grad_W, row_lse, row_kl, workspace, workspace_bytes, status_dev, stream, events);
}

static int32_t fwd_impl(const void* hidden, const void* W, int32_t in_dtype, const int32_t* teacher_idx,
                        const float* teacher_logit, const uint8_t* mask, int64_t T, int64_t d, int64_t V, int64_t K,
                        float tau, int64_t chunk, float* loss, float* row_lse, float* row_kl, void* workspace,
                        size_t workspace_bytes, int32_t* status_dev, void* stream, void* const* events) {
  if (!hidden || !W || !teacher_idx || !teacher_logit || !loss || !row_lse) return KD_ERR_NULL_ARG;
  kd::Args a{hidden, W, teacher_idx, teacher_logit, mask, tau, loss, row_lse, row_kl, nullptr, nullptr, KD_F32,
             nullptr, 0, nullptr, status_dev, (hipStream_t)stream, events};
  return kd::dispatch(kd::kForward, in_dtype, T, d, V, K, chunk, workspace, workspace_bytes, a);
}

int32_t kd_topk_kl_fwd(const void* hidden, const void* W, int32_t in_dtype, const int32_t* teacher_idx,
                       const float* teacher_logit, const uint8_t* mask, int64_t T, int64_t d, int64_t V, int64_t K,
                       float tau, int64_t chunk, float* loss, float* row_lse, float* row_kl, void* workspace,
                       size_t workspace_bytes, int32_t* status_dev, void* stream) {
  return fwd_impl(hidden, W, in_dtype, teacher_idx, teacher_logit, mask, T, d, V, K, tau, chunk, loss, row_lse,
                  row_kl, workspace, workspace_bytes, status_dev, stream, nullptr);
}

int32_t kd_topk_kl_fwd_timed(const void* hidden, const void* W, int32_t in_dtype, const int32_t* teacher_idx,
                             const float* teacher_logit, const uint8_t* mask, int64_t T, int64_t d, int64_t V,
                             int64_t K, float tau, int64_t chunk, float* loss, float* row_lse, float* row_kl,
                             void* workspace, size_t workspace_bytes, int32_t* status_dev, void* stream,
                             void* const* events) {
  if (!events) return KD_ERR_NULL_ARG;
  return fwd_impl(hidden, W, in_dtype, teacher_idx, teacher_logit, mask, T, d, V, K, tau, chunk, loss, row_lse,
                  row_kl, workspace, workspace_bytes, status_dev, stream, events);
}

static int32_t bwd_impl(const void* hidden, const void* W, int32_t in_dtype, const int32_t* teacher_idx,
                        const float* teacher_logit, const uint8_t* mask, int64_t T, int64_t d, int64_t V, int64_t K,
                        float tau, int64_t chunk, const float* row_lse, const float* grad_loss, void* grad_hidden,
                        int32_t grad_hidden_dtype, float* grad_W, int32_t accumulate_grad_W, uint16_t* grad_W_bf16,
                        void* workspace, size_t workspace_bytes, int32_t* status_dev, void* stream,
                        void* const* events) {
  if (!hidden || !W || !teacher_idx || !teacher_logit || !row_lse) return KD_ERR_NULL_ARG;
  if (!grad_hidden && !grad_W) return KD_ERR_NULL_ARG;
  if (grad_W_bf16 && !grad_W) return KD_ERR_NULL_ARG;
  if (grad_hidden_dtype != KD_F32 && grad_hidden_dtype != KD_BF16) return KD_ERR_DTYPE;
  kd::Args a{hidden, W, teacher_idx, teacher_logit, mask, tau, nullptr, const_cast<float*>(row_lse), nullptr,
             grad_loss, grad_hidden, grad_hidden_dtype, grad_W, accumulate_grad_W ? 1 : 0, grad_W_bf16, status_dev,
             (hipStream_t)stream, events};
  return kd::dispatch(kd::kBackward, in_dtype, T, d, V, K, chunk, workspace, workspace_bytes, a);
}

int32_t kd_topk_kl_bwd(const void* hidden, const void* W, int32_t in_dtype, const int32_t* teacher_idx,
                       const float* teacher_logit, const uint8_t* mask, int64_t T, int64_t d, int64_t V, int64_t K,
                       float tau, int64_t chunk, const float* row_lse, const float* grad_loss, void* grad_hidden,
                       int32_t grad_hidden_dtype, float* grad_W, int32_t accumulate_grad_W, uint16_t* grad_W_bf16,
                       void* workspace, size_t workspace_bytes, int32_t* status_dev, void* stream) {
  return bwd_impl(hidden, W, in_dtype, teacher_idx, teacher_logit, mask, T, d, V, K, tau, chunk, row_lse, grad_loss,
                  grad_hidden, grad_hidden_dtype, grad_W, accumulate_grad_W, grad_W_bf16, workspace,
                  workspace_bytes, status_dev, stream, nullptr);
}

int32_t kd_topk_kl_bwd_timed(const void* hidden, const void* W, int32_t in_dtype, const int32_t* teacher_idx,
                             const float* teacher_logit, const uint8_t* mask, int64_t T, int64_t d, int64_t V,
                             int64_t K, float tau, int64_t chunk, const float* row_lse, const float* grad_loss,
                             void* grad_hidden, int32_t grad_hidden_dtype, float* grad_W, int32_t accumulate_grad_W,
                             uint16_t* grad_W_bf16, void* workspace, size_t workspace_bytes, int32_t* status_dev,
                             void* stream, void* const* events) {
  if (!events) return KD_ERR_NULL_ARG;
  return bwd_impl(hidden, W, in_dtype, teacher_idx, teacher_logit, mask, T, d, V, K, tau, chunk, row_lse, grad_loss,
                  grad_hidden, grad_hidden_dtype, grad_W, accumulate_grad_W, grad_W_bf16, workspace,
                  workspace_bytes, status_dev, stream, events);
}

size_t kd_topk_cache_workspace_bytes(int64_t T, int64_t d, int64_t V, int64_t K, int64_t chunk, int32_t in_dtype) {
  kd::CachePlan p;
  if (kd::make_cache_plan(T, d, V, K, chunk, in_dtype, &p) != KD_OK) return 0;
  return p.total;
}

static int32_t cache_impl(const void* hidden, const void* W, int32_t in_dtype, int64_t T, int64_t d, int64_t V,
                          int64_t K, int64_t chunk, int32_t* out_idx, float* out_logit, void* workspace,
                          size_t workspace_bytes, void* stream, void* const* events) {
  if (!hidden || !W || !out_idx || !out_logit) return KD_ERR_NULL_ARG;
  kd::CachePlan p;
  const int32_t st = kd::make_cache_plan(T, d, V, K, chunk, in_dtype, &p);
  if (st != KD_OK) return st;
  if ((((uintptr_t)hidden) | ((uintptr_t)W)) & 15) return KD_ERR_BAD_SHAPE;
  if (!workspace || workspace_bytes < p.total || (((uintptr_t)workspace) & 255)) return KD_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  if (in_dtype == KD_BF16)
    return kd::run_cache<kd::Bf16>(p, hidden, W, out_idx, out_logit, (char*)workspace, s, events);
  return kd::run_cache<kd::F32>(p, hidden, W, out_idx, out_logit, (char*)workspace, s, events);
}

int32_t kd_topk_cache_build(const void* hidden, const void* W, int32_t in_dtype, int64_t T, int64_t d, int64_t V,
                            int64_t K, int64_t chunk, int32_t* out_idx, float* out_logit, void* workspace,
                            size_t workspace_bytes, void* stream) {
  return cache_impl(hidden, W, in_dtype, T, d, V, K, chunk, out_idx, out_logit, workspace, workspace_bytes, stream,
                    nullptr);
}

int32_t kd_topk_cache_build_timed(const void* hidden, const void* W, int32_t in_dtype, int64_t T, int64_t d,
                                  int64_t V, int64_t K, int64_t chunk, int32_t* out_idx, float* out_logit,
                                  void* workspace, size_t workspace_bytes, void* stream, void* const* events) {
  if (!events) return KD_ERR_NULL_ARG;
  return cache_impl(hidden, W, in_dtype, T, d, V, K, chunk, out_idx, out_logit, workspace, workspace_bytes, stream,
                    events);
}

int32_t kd_mfma_probe(int32_t blocks, int32_t iters, int32_t zero_operands, float* out, void* stream) {
  if (!out) return KD_ERR_NULL_ARG;
  if (blocks < 1 || iters < 1) return KD_ERR_BAD_SHAPE;
  hipLaunchKernelGGL(kd::mfma_probe_kernel, dim3((unsigned)blocks), dim3(512), 0, (hipStream_t)stream, (int)iters,
                     zero_operands ? 1 : 0, out);
  return hipGetLastError() == hipSuccess ? KD_OK : KD_ERR_HIP;
}

const char* kd_status_str(int32_t s) {
  switch (s) {
    case KD_OK: return "ok";
    case KD_ERR_NULL_ARG: return "a required pointer is NULL";
    case KD_ERR_BAD_SHAPE: return "bad shape (T, d, V, K < 1, K > V, K > KD_MAX_K, too large, or misaligned input)";
    case KD_ERR_BAD_TAU: return "tau must be finite and > 0";
    case KD_ERR_BAD_CHUNK: return "chunk must be >= 1";
    case KD_ERR_DTYPE: return "in_dtype (or the gradient output dtype) must be KD_BF16 or KD_F32";
    case KD_ERR_WORKSPACE: return "workspace is NULL, too small or not 256-byte aligned";
    case KD_ERR_BAD_INDEX: return "a teacher id is outside [0, V)";
    case KD_ERR_HIP: return "a HIP launch failed";
    case KD_ERR_NOALLOC_SIZE:
      return "the sizes need more workspace than the allocation-free entry point's fixed device scratch "
             "(KD_NOALLOC_SCRATCH_BYTES) holds";
    default: return "unknown status";
  }
}

}  // extern "C"
