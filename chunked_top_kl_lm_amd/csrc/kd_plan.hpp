// kd_plan.hpp -- host-side plan of a call: tile configurations, argument
// and addressing limits, and the workspace carve-up of the loss's entry points
// and of the cache builder.  Plain C++ (no HIP types), so that the host
// checks (tests/index_check.cpp) build it with a host compiler and address
// sanitizer and sweep it over shapes.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <algorithm>

#include "../../include/kd_topk_kl.h"
#include "kd_layout.hpp"

namespace kd {

// GEMM tile configurations (block tile BM x BN, WM x WN waves, STAGES LDS
// stages of RB bytes of K), chosen by measurement on MI355X:
//  - the logit GEMMs: 256 x 256, 8 waves of 128 x 64, 2 stages of 128 bytes
//    (128 KB LDS, one block per CU; half the barriers of 64-byte stages);
//  - the hidden-gradient GEMM (N = d): 256 x 256, or 256 x 320 (8 waves of
//    64 x 160, 144 KB LDS) when that pads d less -- at d = 2880 the 320-wide
//    tile covers d exactly where 256 wastes 6% of the columns;
//  - the head-gradient GEMM (N = d, fp32 read-modify-write epilogue):
//    256 x 320 when that pads d no more than the alternatives (its epilogue
//    updates 96 of a wave's 160 columns from the accumulators and the rest
//    through LDS with 16-byte accesses; d a multiple of 4), else 256 x 192
//    (8 waves of 64 x 96, 112 KB LDS) or 256 x 128, whichever pads d less.
//    Those keep all grad_W loads of a wave in flight at once.
template <int BM_, int BN_, int WM_, int WN_, int ST_, int RB_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, STAGES = ST_, RB = RB_;
  static constexpr int kThreads = 64 * WM * WN;
};
using TileMain = TileCfg<256, 256, 2, 4, 2, 128>;
using TileDhWide = TileCfg<256, 320, 4, 2, 2, 128>;
using TileHead = TileCfg<256, 192, 4, 2, 2, 128>;
using TileHeadNarrow = TileCfg<256, 128, 4, 2, 2, 128>;
constexpr int kBM = TileMain::BM, kBN = TileMain::BN;
constexpr int kWaveM = TileMain::BM / TileMain::WM;   // vocabulary strip of one LSE partial
constexpr int kNumCU = 256;           // MI355X compute units (split-K sizing)
// The head-gradient GEMM contracts over at least this many rows per launch
// (several consecutive chunks when the chunk is smaller): each launch reads
// and writes the whole fp32 grad_W once, so fewer, longer launches cut that
// traffic.  At 2048-row chunks (d = 2880, V = 201088) 4096 rows per launch
// took 2.19 vs 2.44 ms per 2048 rows for one chunk, and 8192 rows take 2 ms
// less per 32K step again (measured against 4096 in the same run), for two
// more chunk-sized G^T buffers (1.65 GB, independent of T).
constexpr int64_t kDwRows = 8192;

inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
inline int64_t cdiv(int64_t x, int64_t m) { return (x + m - 1) / m; }
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// What a call computes: the fused forward + backward, the forward alone
// (loss and the saved per-row logsumexp), or the backward alone (recomputed
// from that logsumexp).
enum Mode { kFused = 0, kForward = 1, kBackward = 2 };

struct Plan {
  int mode;
  bool fwd, bwd;      // the call runs the forward steps / the backward steps
  int64_t T, d, V, K, chunk, nchunks;
  int eb;             // element bytes
  bool pad_d;         // d is not a multiple of 64: use zero-padded copies
  int64_t d_p, V_p, R_p, Nd_p;
  int dh_bn, dw_bn;   // column tile (over d) of the hidden- and head-gradient GEMMs
  bool dw_wide;       // head-gradient GEMM on 256 x 320 tiles (LDS-staged update)
  int dw_group;       // consecutive chunks whose G^T and H_c^T one head-gradient GEMM contracts
  int64_t R_g;        // dw_group * R_p: row stride of the G^T and H_c^T buffers
  int64_t nvt;        // LSE strips per row
  int splits;         // split-K factor of the hidden-gradient GEMM
  int64_t nbt;        // teacher-id hit lists: row groups per chunk
  int64_t ng;         // first-level LSE merge groups per row
  // workspace offsets (buffers a mode does not use take no space)
  size_t off_scalar, off_wt, off_wp, off_hp, off_ht, off_g, off_gt, off_part, off_lse2, off_rowkl, off_dh;
  size_t off_hoff, off_hits, off_zsel, off_part2, off_psel;
  size_t total;
};

// lean: one chunk per head-gradient launch (the smallest workspace; used by
// the allocation-free entry point, whose workspace is a fixed static array).
inline int32_t make_plan(int64_t T, int64_t d, int64_t V, int64_t K, int64_t chunk, int32_t dt, int mode, Plan* p,
                  bool lean = false) {
  if (dt != KD_BF16 && dt != KD_F32) return KD_ERR_DTYPE;
  if (T < 1 || d < 1 || V < 1 || K < 1 || K > V || K > KD_MAX_K) return KD_ERR_BAD_SHAPE;
  if (chunk < 1) return KD_ERR_BAD_CHUNK;
  Plan& P = *p;
  P.mode = mode;
  P.fwd = mode != kBackward;
  P.bwd = mode != kForward;
  P.T = T; P.d = d; P.V = V; P.K = K;
  P.chunk = chunk > T ? T : chunk;
  P.nchunks = cdiv(T, P.chunk);
  P.eb = dt == KD_BF16 ? 2 : 4;
  P.pad_d = (d % 64) != 0;
  P.d_p = round_up(d, 64);
  P.V_p = round_up(V, kBM);
  P.R_p = round_up(P.chunk, kBN);
  P.dh_bn = round_up(d, TileDhWide::BN) < round_up(d, TileMain::BN) ? TileDhWide::BN : TileMain::BN;
  P.dw_bn = round_up(d, TileHead::BN) <= round_up(d, TileHeadNarrow::BN) ? TileHead::BN : TileHeadNarrow::BN;
  P.dw_wide = d % 4 == 0 && round_up(d, TileDhWide::BN) <= round_up(d, P.dw_bn);
  P.Nd_p = round_up(d, P.dh_bn);
  P.nvt = P.V_p / kWaveM;
  P.dw_group = P.bwd && !lean ? (int)std::max<int64_t>(1, std::min<int64_t>(P.nchunks, kDwRows / P.R_p)) : 1;
  P.R_g = P.dw_group * P.R_p;
  P.nbt = P.R_p / kHitT;
  P.ng = cdiv(P.nvt, kMergeStrips);
  // Addressing limits: per-tile buffer ranges and int32 tile indices.
  if (P.V_p > (1ll << 24) || P.d_p > (1ll << 20) || P.R_g > (1ll << 20) || T > (1ll << 31) / 2)
    return KD_ERR_BAD_SHAPE;
  if ((int64_t)kBM * P.V_p * P.eb >= (1ll << 32) || (int64_t)kBM * P.R_g * P.eb >= (1ll << 32))
    return KD_ERR_BAD_SHAPE;
  // hit lists: int32 entry indices; a row group's strip counts sit in 64 KB
  // of LDS, so V_p / 128 + 1 <= 16384, i.e. V <= 2096896
  if (P.R_p * K >= (1ll << 31) || (P.nvt + 1) * 4 > 65536) return KD_ERR_BAD_SHAPE;
  // split-K of the hidden-gradient GEMM (output only chunk x d): pick the
  // split count whose grid fills whole waves of 256 CUs best, with at least
  // one full wave, and a small penalty per split for the partial-sum traffic.
  const int64_t tiles = cdiv(P.R_p, kBM) * (P.Nd_p / P.dh_bn);
  const int64_t k_tiles = P.V_p * P.eb / TileMain::RB;
  int best = 1;
  double best_cost = 1e30;
  for (int sp = 1; sp <= 64 && sp <= k_tiles; ++sp) {
    const int64_t blocks = tiles * sp;
    const double waves = (double)blocks / kNumCU;
    double cost = (double)cdiv(blocks, kNumCU) / waves + 0.004 * sp;
    if (blocks < kNumCU) cost += 1.0;                      // too little parallelism
    if (k_tiles / sp < 16) cost += 1.0;                     // splits too thin
    if (cost < best_cost) { best_cost = cost; best = sp; }
  }
  // every split must own at least one K stage
  const int64_t kps = cdiv(k_tiles, best);
  P.splits = (int)cdiv(k_tiles, kps);

  const size_t e = (size_t)P.eb;
  const bool F = P.fwd, B = P.bwd;
  size_t o = 0;
  auto take = [&](size_t& off, bool used, size_t bytes) {
    off = o;
    if (used) o = align256(o + bytes);
  };
  P.off_scalar = o; o += 256;
  take(P.off_wt, B, (size_t)P.d_p * P.V_p * e);
  take(P.off_wp, P.pad_d, (size_t)V * P.d_p * e);
  take(P.off_hp, P.pad_d, (size_t)P.R_p * P.d_p * e);
  take(P.off_ht, B, (size_t)P.d_p * P.R_g * e);
  take(P.off_g, B, (size_t)P.R_p * P.V_p * e);
  take(P.off_gt, B, (size_t)P.V_p * P.R_g * e);
  take(P.off_part, F, (size_t)P.nvt * P.R_p * (2 * sizeof(float)));
  take(P.off_lse2, F, (size_t)P.R_p * sizeof(float));
  take(P.off_rowkl, F, (size_t)P.R_p * sizeof(double));
  take(P.off_dh, B, (size_t)P.splits * P.R_p * P.Nd_p * sizeof(float));
  take(P.off_hoff, true, (size_t)P.nbt * (P.nvt + 1) * sizeof(int));
  take(P.off_hits, true, (size_t)P.R_p * K * (2 * sizeof(uint32_t)));
  take(P.off_zsel, F, (size_t)P.R_p * K * sizeof(float));
  take(P.off_part2, F, (size_t)P.ng * P.R_p * (2 * sizeof(float)));
  take(P.off_psel, B, (size_t)P.R_p * K * sizeof(float));   // teacher p for the epilogue's sparse part
  P.total = o;
  return KD_OK;
}


inline size_t workspace_for(int mode, int64_t T, int64_t d, int64_t V, int64_t K, int64_t chunk, int32_t in_dtype) {
  Plan p;
  if (make_plan(T, d, V, K, chunk, in_dtype, mode, &p) != KD_OK) return 0;
  return p.total;
}

// ---------------------------------------------------------------------------
// Offline top-K cache builder (see kd_cache.hpp)
// ---------------------------------------------------------------------------
struct CachePlan {
  int64_t T, d, V, K, chunk, nchunks;
  int eb;
  bool pad_d;
  int64_t d_p, V_p, R_p;
  int64_t nb32;       // 32-row vocabulary blocks with a valid row
  int cap;            // candidate list length per row (power of two)
  int half;           // fallback: power of two >= max(K, batch)
  size_t off_wp, off_hp, off_bmax, off_theta, off_cnt, off_cand, off_ovf, off_z, total;
};

inline int pow2ceil(int64_t x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

inline int32_t make_cache_plan(int64_t T, int64_t d, int64_t V, int64_t K, int64_t chunk, int32_t dt, CachePlan* p) {
  if (dt != KD_BF16 && dt != KD_F32) return KD_ERR_DTYPE;
  if (T < 1 || d < 1 || V < 1 || K < 1 || K > V || K > KD_MAX_K) return KD_ERR_BAD_SHAPE;
  if (chunk < 1) return KD_ERR_BAD_CHUNK;
  CachePlan& P = *p;
  P.T = T; P.d = d; P.V = V; P.K = K;
  P.chunk = chunk > T ? T : chunk;
  P.nchunks = cdiv(T, P.chunk);
  P.eb = dt == KD_BF16 ? 2 : 4;
  P.pad_d = (d % 64) != 0;
  P.d_p = round_up(d, 64);
  P.V_p = round_up(V, kBM);
  P.R_p = round_up(P.chunk, kBN);
  if (P.V_p > (1ll << 24) || P.d_p > (1ll << 20) || P.R_p > (1ll << 20) || T > (1ll << 31) / 2)
    return KD_ERR_BAD_SHAPE;
  if ((int64_t)kBM * P.V_p * P.eb >= (1ll << 32) || (int64_t)kBM * P.R_p * P.eb >= (1ll << 32))
    return KD_ERR_BAD_SHAPE;
  P.nb32 = cdiv(V, kBlockRows);
  // Candidate list: twice K (rounded up to a power of two), at least 256;
  // when there are fewer blocks than K every logit is a candidate, so the
  // list must hold V.  Past 8192 (64 KB of sort keys) rows go to the
  // fallback.
  int64_t want = std::max<int64_t>(2 * K, 256);
  if (P.nb32 < K) want = std::max<int64_t>(want, V);
  P.cap = pow2ceil(std::min<int64_t>(want, 8192));
  P.half = pow2ceil(std::max<int64_t>(K, kFbBatch));
  const size_t e = (size_t)P.eb;
  size_t o = 0;
  P.off_wp = o; if (P.pad_d) o = align256(o + (size_t)V * P.d_p * e);
  P.off_hp = o; if (P.pad_d) o = align256(o + (size_t)P.R_p * P.d_p * e);
  P.off_bmax = o; o = align256(o + (size_t)P.R_p * (P.V_p / kBlockRows) * sizeof(float));   // [R_p][V_p/32]
  P.off_theta = o; o = align256(o + (size_t)P.R_p * sizeof(float));
  P.off_cnt = o; o = align256(o + (size_t)P.R_p * sizeof(int));
  P.off_cand = o; o = align256(o + (size_t)P.R_p * P.cap * (2 * sizeof(uint32_t)));
  P.off_ovf = o; o = align256(o + (size_t)P.R_p * sizeof(int));
  P.off_z = o; o = align256(o + (size_t)P.R_p * P.V_p * sizeof(float));                   // [R_p][V_p] logits
  P.total = o;
  return KD_OK;
}

}  // namespace kd
