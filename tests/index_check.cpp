// index_check.cpp -- host checks of the kernels' index arithmetic and of the
// workspace carve-up, built with a host compiler under the address and
// undefined-behaviour sanitizers (tests/test_index_math.py).
//
// It includes the library's own kd_layout.hpp (every address the GEMM
// epilogues, the hit lists and the operand staging form) and kd_plan.hpp
// (the plan and workspace offsets), and sweeps ragged shapes:
//   accumulator layout: acc_row/acc_col is a bijection onto 32x32 and
//     acc_reg_of/acc_lane_of invert it (the hit walks rely on it);
//   hit codes round-trip (v % 128, t % 64);
//   head-gradient RMW (EpiAccum, all three tile widths, the LDS-staged
//     columns of the 320-wide tile): every in-range element lands on its own
//     (m, n) inside the wave's buffer resource, every out-of-range one
//     (rows >= V, columns >= d) falls outside it, no 32-bit offset wraps, the
//     staging covers the wave's 64 x 64 block once and stays in its LDS slice;
//   gradient staging (EpiGrad): both LDS layouts are written once per
//     element and every 16-byte read returns 8 consecutive elements of one
//     row; the global stores stay inside G [R_p][V_p] and the chunk's slot of
//     G^T [V_p][R_g];
//   logsumexp partials and hit-list bounds stay inside their buffers;
//   operand staging: DMA offsets of valid rows fit the K extent and resource;
//   cache builder: the logit staging writes each (t, v) once and every read
//     returns 4 consecutive v of one row; the 16-byte logit stores land on
//     their own (t, v) inside [R_p][V_p] and cover a wave tile once; the collect
//     loads stay inside a row; the cache plan's buffers are aligned,
//     ordered, disjoint and inside the total;
//   plan: for every mode, buffers are 256-byte aligned, ordered, disjoint,
//     inside the total, and at least as large as the kernels index them; a
//     host buffer of exactly `total` bytes is written region by region (the
//     sanitizer catches a region past the end).
// `--plant NAME` reintroduces one plausible mistake; the run must then fail.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <set>
#include <string>
#include <vector>

#include "kd_plan.hpp"

using namespace kd;

static std::string g_plant;
static long g_checks = 0, g_fail = 0;

#define CHECK(cond, ...)                                  \
  do {                                                    \
    ++g_checks;                                           \
    if (!(cond)) {                                        \
      if (g_fail < 12) {                                  \
        fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
        fprintf(stderr, __VA_ARGS__);                     \
        fprintf(stderr, "\n");                            \
      }                                                   \
      ++g_fail;                                           \
    }                                                     \
  } while (0)

static bool planted(const char* name) { return g_plant == name; }

// ---------------------------------------------------------------------------
static void check_acc_layout() {
  std::set<int> seen;
  for (int lane = 0; lane < 64; ++lane)
    for (int r = 0; r < 16; ++r) {
      const int rr = acc_row(r, lane), col = acc_col(lane);
      CHECK(rr >= 0 && rr < 32 && col >= 0 && col < 32, "acc (%d,%d) out of tile", rr, col);
      seen.insert(rr * 32 + col);
      CHECK(acc_reg_of(rr) == r && acc_lane_of(rr, col) == lane, "acc inverse r=%d lane=%d", r, lane);
    }
  CHECK(seen.size() == 1024, "accumulator layout covers %zu of 1024", seen.size());
}

static void check_hit_codes() {
  for (int v = 0; v < 4 * kHitV; v += 3)
    for (int t = 0; t < kHitT; ++t) {
      const uint32_t h = hit_code(v, t);
      CHECK(h < (1u << 13) && hit_code_v(h) == v % kHitV && hit_code_t(h) == t, "hit code v=%d t=%d", v, t);
    }
}

// ---------------------------------------------------------------------------
// Head gradient: grad_W [M = V][N = d], ld = d floats, wave tiles 64 x (32 FN)
// of BM x BN blocks (4 x 2 waves).  `wide`: FN = 5, columns 96..159 via LDS.
static void check_accum(int M, int N, int BN, bool wide, int lds_slice_bytes) {
  const int FM = 2, FN = BN / 2 / 32;
  const int64_t ld = N;
  const uint32_t ld4 = (uint32_t)ld * 4u;
  const int tiles_m = (M + 255) / 256, tiles_n = (N + BN - 1) / BN;
  std::vector<int> tms;
  std::vector<int> tns;
  for (int tm = 0; tm < tiles_m; ++tm)
    if (tm < 2 || tm >= tiles_m - 2) tms.push_back(tm);
  for (int tn = 0; tn < tiles_n; ++tn)
    if (tn < 2 || tn >= tiles_n - 2) tns.push_back(tn);
  const int guard_M = planted("accum-row-guard") ? tiles_m * 256 : M;
  const int guard_N = planted("accum-col-guard") ? (1 << 30) : N;
  for (int tm : tms)
    for (int tn : tns)
      for (int wid = 0; wid < 8; ++wid) {
        const int wm = wid / 2, wn = wid % 2;
        const int m0 = tm * 256 + wm * 64, n0 = tn * BN + wn * (BN / 2);
        const int rows = accum_rows(m0, 64, guard_M);
        const uint64_t bytes = (uint64_t)rows * ld * 4;
        CHECK(bytes < (1ull << 32), "resource bytes %llu", (unsigned long long)bytes);
        const int direct = wide ? 3 : FN;
        std::vector<int> staged(64 * 64, 0);
        for (int lane = 0; lane < 64; ++lane) {
          for (int j = 0; j < FN; ++j) {
            const int n = n0 + 32 * j + acc_col(lane);
            const uint32_t vo = accum_lane_offset(n, guard_N, lane, ld4);
            for (int i = 0; i < FM; ++i)
              for (int r = 0; r < 16; ++r) {
                const int m = m0 + 32 * i + acc_row(r, lane);
                if (j >= direct) {
                  const int idx = wide_stage_index(i, j, r, lane);
                  CHECK(idx >= 0 && (idx + 1) * 4 <= lds_slice_bytes && idx < 64 * kWideStride, "wide stage %d", idx);
                  const int sr = idx / kWideStride, sc = idx % kWideStride;
                  CHECK(sr == 32 * i + acc_row(r, lane) && sc == 32 * (j - 3) + acc_col(lane), "wide stage map");
                  if (sr < 64 && sc < 64) staged[sr * 64 + sc]++;
                  continue;
                }
                const uint64_t off64 = (uint64_t)vo + (uint64_t)(acc_row(r, 0) + 32 * i) * ld4;
                const uint32_t off = accum_elem_offset(vo, i, r, ld4);
                CHECK(off64 == off, "offset wraps m0=%d n=%d", m0, n);
                if (m < M && n < N) {
                  CHECK((uint64_t)off + 4 <= bytes, "in-range element outside resource m=%d n=%d", m, n);
                  CHECK(off == (uint64_t)(m - m0) * ld * 4 + (uint64_t)n * 4, "element misaddressed m=%d n=%d", m, n);
                } else {
                  CHECK((uint64_t)off + 4 > bytes, "element past the matrix lands inside m=%d n=%d (M=%d N=%d)", m, n,
                        M, N);
                }
              }
          }
        }
        if (!wide) continue;
        for (int k = 0; k < 64 * 64; ++k) CHECK(staged[k] == 1, "wide staging element %d written %d times", k, staged[k]);
        std::vector<int> read(64 * 64, 0);
        for (int lane = 0; lane < 64; ++lane) {
          const int col = wide_read_col(lane);
          const int n = n0 + 96 + col;
          const uint32_t vs = wide_lane_offset(n, guard_N, lane, ld4);
          for (int q = 0; q < 16; ++q) {
            const int row = wide_read_row(q, lane);
            CHECK(row < 64 && col + 3 < 64, "wide read (%d,%d)", row, col);
            CHECK(((row * kWideStride + col) * 4) % 16 == 0 && (row * kWideStride + col + 4) * 4 <= lds_slice_bytes,
                  "wide read alignment/slice");
            for (int e = 0; e < 4; ++e) read[row * 64 + col + e]++;
            const int m = m0 + row;
            const uint64_t off64 = (uint64_t)vs + (uint64_t)(4 * q) * ld4;
            const uint32_t off = wide_elem_offset(vs, q, ld4);
            CHECK(off64 == off, "wide offset wraps");
            if (m < M && n < N) {
              CHECK(n + 3 < N, "16-byte access straddles N (N %% 4 = %d)", N % 4);
              CHECK((uint64_t)off + 16 <= bytes, "wide element outside resource m=%d n=%d", m, n);
              CHECK(off == (uint64_t)(m - m0) * ld * 4 + (uint64_t)n * 4, "wide element misaddressed");
            } else {
              CHECK((uint64_t)off + 16 > bytes, "wide element past the matrix lands inside m=%d n=%d", m, n);
            }
          }
        }
        for (int k = 0; k < 64 * 64; ++k) CHECK(read[k] == 1, "wide staging element %d read %d times", k, read[k]);
      }
}

// ---------------------------------------------------------------------------
// Gradient staging: simulate both layouts in a 16 KB slice.
static void check_grad_staging() {
  std::vector<int> tag(kGradStageBytes / 2, -1);   // bf16 slots
  for (int lane = 0; lane < 64; ++lane)
    for (int j = 0; j < 2; ++j)
      for (int i = 0; i < 4; ++i)
        for (int g4 = 0; g4 < 4; ++g4) {
          const int tl = 32 * j + acc_col(lane);
          const int vl0 = 32 * i + 8 * g4 + 4 * (lane >> 5);
          int off = g_stage_offset(tl, vl0);
          if (planted("g-stage-swizzle")) off = tl * 256 + ((vl0 >> 3) << 4) + ((vl0 & 7) << 1);
          CHECK(off >= 0 && off % 8 == 0 && off + 8 <= kGradStageBytes, "G stage offset %d", off);
          for (int e = 0; e < 4; ++e) {
            CHECK(tag[off / 2 + e] == -1, "G staging slot written twice");
            tag[off / 2 + e] = tl * 128 + vl0 + e;
          }
        }
  for (int q = 0; q < 16; ++q)
    for (int lane = 0; lane < 64; ++lane) {
      const int off = g_read_offset(q, lane), t = g_read_row(q, lane), u = g_read_unit(lane);
      CHECK(off % 16 == 0 && off + 16 <= kGradStageBytes, "G read offset %d", off);
      for (int e = 0; e < 8; ++e) CHECK(tag[off / 2 + e] == t * 128 + 8 * u + e, "G read q=%d lane=%d e=%d", q, lane, e);
    }
  std::fill(tag.begin(), tag.end(), -1);
  for (int lane = 0; lane < 64; ++lane)
    for (int j = 0; j < 2; ++j)
      for (int i = 0; i < 4; ++i)
        for (int g4 = 0; g4 < 4; ++g4)
          for (int e = 0; e < 4; ++e) {
            const int tl = 32 * j + acc_col(lane);
            const int vl = 32 * i + 8 * g4 + 4 * (lane >> 5) + e;
            const int off = gt_stage_offset(vl, tl);
            CHECK(off >= 0 && off % 2 == 0 && off + 2 <= kGradStageBytes, "G^T stage offset %d", off);
            CHECK(tag[off / 2] == -1, "G^T staging slot written twice");
            tag[off / 2] = vl * 64 + tl;
          }
  for (int q = 0; q < 16; ++q)
    for (int lane = 0; lane < 64; ++lane) {
      const int off = gt_read_offset(q, lane), v = gt_read_row(q, lane), u = gt_read_unit(lane);
      CHECK(off % 16 == 0 && off + 16 <= kGradStageBytes, "G^T read offset %d", off);
      for (int e = 0; e < 8; ++e) CHECK(tag[off / 2 + e] == v * 64 + 8 * u + e, "G^T read q=%d lane=%d", q, lane);
    }
}

// ---------------------------------------------------------------------------
// Per-plan checks: the global ranges the per-chunk kernels index, against the
// buffers the plan carves out.
struct Buf {
  const char* name;
  size_t off;
  size_t need;   // bytes the kernels index
  bool used;
};

static void check_plan(int64_t T, int64_t d, int64_t V, int64_t K, int64_t chunk, int dt, int mode, bool lean) {
  Plan P;
  const int32_t st = make_plan(T, d, V, K, chunk, dt, mode, &P, lean);
  if (st != KD_OK) return;
  const size_t eb = (size_t)P.eb;
  const bool F = P.fwd, B = P.bwd;
  const int64_t R_g_kernel = P.R_g;   // the stride the epilogue and the GEMM use
  const int64_t R_g_buf = planted("gt-group-stride") ? P.R_p : P.R_g;
  // what the kernels index in each buffer
  std::vector<Buf> bufs = {
      {"W^T", P.off_wt, (size_t)P.d_p * P.V_p * eb, B},
      {"W pad", P.off_wp, (size_t)V * P.d_p * eb, P.pad_d},
      {"H pad", P.off_hp, (size_t)P.R_p * P.d_p * eb, P.pad_d},
      {"H^T", P.off_ht, (size_t)P.d_p * R_g_kernel * eb, B},
      {"G", P.off_g, (size_t)P.R_p * P.V_p * eb, B},
      {"G^T", P.off_gt, (size_t)P.V_p * R_g_kernel * eb, B},
      {"LSE partials", P.off_part, (size_t)P.nvt * P.R_p * 8, F},
      {"lse2", P.off_lse2, (size_t)P.R_p * 4, F},
      {"row KL", P.off_rowkl, (size_t)P.R_p * 8, F},
      {"dH partials", P.off_dh, (size_t)P.splits * P.R_p * P.Nd_p * 4, B},
      {"hit offsets", P.off_hoff, (size_t)P.nbt * (P.nvt + 1) * 4, true},
      {"hit entries", P.off_hits, (size_t)P.R_p * K * 8, true},
      {"z at ids", P.off_zsel, (size_t)P.R_p * K * 4, F},
      {"LSE group partials", P.off_part2, (size_t)P.ng * P.R_p * 8, F},
      {"teacher p", P.off_psel, (size_t)P.R_p * K * 4, B},
  };
  if (planted("gt-group-stride")) bufs[5].need = (size_t)P.V_p * R_g_buf * eb;   // (kept consistent below)
  CHECK(P.off_scalar == 0 && P.total >= 256, "scalars");
  size_t prev_end = 256;
  for (const Buf& b : bufs) {
    if (!b.used) continue;
    CHECK(b.off % 256 == 0, "%s not 256-byte aligned", b.name);
    CHECK(b.off >= prev_end, "%s overlaps the previous buffer", b.name);
    CHECK(b.off + b.need <= P.total, "%s ends past the workspace (%zu + %zu > %zu)", b.name, b.off, b.need, P.total);
    prev_end = b.off + b.need;
  }
  // the chunk's slot of G^T: the epilogue writes columns gslot*R_p + [0, Rt)
  // of rows [0, V_p) with row stride R_g; the buffer holds V_p * R_g_buf
  if (B) {
    const int64_t gslot_max = P.dw_group - 1;
    const int64_t last_col = gslot_max * P.R_p + P.R_p;                 // exclusive
    CHECK(last_col <= R_g_kernel, "G^T slot past the row");
    CHECK((uint64_t)(P.V_p - 1) * R_g_kernel + last_col <= (uint64_t)P.V_p * R_g_buf,
          "G^T slot %lld past the buffer (R_g %lld)", (long long)gslot_max, (long long)R_g_buf);
    // G stores: rows n0 + t < R_p, columns m0 + 8u + 8 <= V_p
    CHECK(P.R_p % kHitT == 0 && P.V_p % kHitV == 0, "wave tiles tile the padded chunk and vocabulary");
  }
  if (F) {
    // EpiLsePartial: part[vt * R_p + n0 + 32 j + lane], vt < nvt
    CHECK((size_t)(P.nvt - 1) * P.R_p + (P.R_p - 1) < (size_t)P.nvt * P.R_p, "LSE partial index");
    // hit-list bounds: b + 1 with b = (n0 / 64) (nvt + 1) + m0 / 128
    const int64_t bmax = (P.R_p / kHitT - 1) * (P.nvt + 1) + (P.V_p / kHitV - 1);
    CHECK(bmax + 1 < P.nbt * (P.nvt + 1), "hit-list bounds index");
    CHECK((P.nvt + 1) * 4 <= 65536, "hit-list strip counts exceed 64 KB of LDS");
  }
  // hit entries: group g owns [g 64 K, (g + 1) 64 K) < R_p K < 2^31
  CHECK(P.nbt * kHitT * K <= P.R_p * K && P.R_p * K < (1ll << 31), "hit entry index range");
  // teacher rows: dynamic LDS + the kernels' static arrays within 64 KB
  CHECK(teacher_lds_bytes((int)K) + 256 * 4 + 256 * 8 <= 65536, "teacher-row LDS for K=%lld", (long long)K);
  // operand staging: K extents are whole 128-byte stages and fit the rows
  const int64_t kb_d = P.d_p * P.eb;
  CHECK(kb_d % TileMain::RB == 0, "forward K extent %lld not whole stages", (long long)kb_d);
  CHECK((int64_t)(P.pad_d ? P.d_p : d) * P.eb >= kb_d, "forward K extent past the operand rows");
  CHECK((uint64_t)kBM * (uint64_t)(P.pad_d ? P.d_p : d) * P.eb < (1ull << 32), "forward operand resource");
  if (B) {
    CHECK((P.V_p * P.eb) % TileMain::RB == 0 && (P.R_g * P.eb) % TileMain::RB == 0, "gradient K extents");
    CHECK((uint64_t)kBM * P.V_p * P.eb < (1ull << 32) && (uint64_t)kBM * P.R_g * P.eb < (1ull << 32),
          "gradient operand resources");
    // the DMA offsets of a stage: row r < BM, unit < RB / 16, plus the stage
    for (int lane = 0; lane < 64; ++lane)
      for (int r = 0; r < 256; r += 37) {
        const uint32_t o = dma_src_offset<128>(r, lane, P.V_p * P.eb);
        CHECK(o >= (uint32_t)(r * P.V_p * P.eb) && o + 16 <= (uint32_t)(r * P.V_p * P.eb + 128), "DMA unit");
      }
  }
  // a host buffer of exactly `total` bytes (small plans), written region by
  // region: a region past the end is a heap overflow the sanitizer reports.
  // The planted mistake: a total that leaves out the last buffer.
  size_t total = P.total, last_off = 0;
  for (const Buf& b : bufs)
    if (b.used) last_off = b.off;
  if (planted("plan-total")) total = last_off;
  if (total <= (4u << 20)) {
    unsigned char* ws = (unsigned char*)malloc(total);
    for (const Buf& b : bufs)
      if (b.used) memset(ws + b.off, 0x5a, b.need);
    free(ws);
  }
}

// ---------------------------------------------------------------------------
// Cache builder: the GEMM epilogue's logit stores and block maxima, the
// collect kernel's row loads, and the cache plan's buffers.
// the logit staging of one wave and column half: every (t, v) written once,
// 16-byte aligned, inside the 16 KB slice, each register at its own (t, v);
// every read returns 4 consecutive v of one row and the reads cover the half
static void check_cache_staging() {
  std::set<int> wr;
  for (int lane = 0; lane < 64; ++lane)
    for (int i = 0; i < 4; ++i)
      for (int g4 = 0; g4 < 4; ++g4) {
        const int tl = acc_col(lane), vl0 = 32 * i + 8 * g4 + 4 * (lane >> 5);
        const int o = cz_stage_offset(tl, vl0);
        CHECK(o % 16 == 0 && o >= 0 && o + 16 <= kCacheStageBytes, "cache staging write %d", o);
        for (int e = 0; e < 4; ++e) {
          CHECK(32 * i + acc_row(4 * g4 + e, lane) == vl0 + e, "cache staging register %d holds v %d",
                4 * g4 + e, vl0 + e);
          wr.insert(o + 4 * e);
        }
      }
  CHECK(wr.size() == 32 * 128, "cache staging writes cover %zu of 4096", wr.size());
  std::set<int> rd;
  for (int q = 0; q < 16; ++q)
    for (int lane = 0; lane < 64; ++lane) {
      const int t = cz_read_row(q, lane), u = cz_read_unit(lane);
      CHECK(t < 32 && u < 32 && cz_read_offset(q, lane) == cz_stage_offset(t, 4 * u), "cache staging read");
      rd.insert(t * 32 + u);
    }
  CHECK(rd.size() == 32 * 32, "cache staging reads cover %zu of 1024 units", rd.size());
  // 8 waves' slices fit the logit GEMM's LDS ring
  CHECK(8 * kCacheStageBytes <= TileMain::STAGES * (TileMain::BM + TileMain::BN) * TileMain::RB, "cache staging LDS");
}

static std::set<std::pair<int64_t, int64_t>> g_cache_tiles_done;

// the global stores of a wave tile at the first and last strip and column
// block: 16-byte aligned, each value at its own (t, v) inside [R_p][V_p],
// the tile covered once (depends on V_p and R_p only; each pair once)
static void check_cache_tiles(int64_t V, int64_t V_p, int64_t R_p) {
  if (!g_cache_tiles_done.insert({V_p, R_p}).second) return;
  const int64_t ldz = planted("cache-z-stride") ? V : V_p;
  const int m0s[] = {0, (int)(V_p - 128)};
  const int n0s[] = {0, (int)(R_p - 64)};
  for (int m0 : m0s)
    for (int n0 : n0s) {
      std::set<int64_t> seen;
      for (int j = 0; j < 2; ++j)
        for (int q = 0; q < 16; ++q)
          for (int lane = 0; lane < 64; ++lane) {
            const int t = n0 + 32 * j + cz_read_row(q, lane), u = cz_read_unit(lane);
            const int64_t o = cz_global_offset(t, ldz, m0, u);
            CHECK(o % 4 == 0, "logit store not 16-byte aligned (V_p %lld)", (long long)V_p);
            for (int e = 0; e < 4; ++e) {
              const int64_t want = (int64_t)t * V_p + m0 + 4 * u + e;
              CHECK(o + e == want, "logit store element (t %d, v %d) at %lld, want %lld", t, m0 + 4 * u + e,
                    (long long)(o + e), (long long)want);
              CHECK(o + e >= 0 && o + e < R_p * V_p, "logit store past the buffer");
              seen.insert(o + e);
            }
          }
      CHECK(seen.size() == 128 * 64, "logit stores cover %zu of a wave tile's 8192", seen.size());
    }
}

static void check_cache_plan(int64_t T, int64_t d, int64_t V, int64_t K, int64_t chunk, int dt) {
  CachePlan P;
  if (make_cache_plan(T, d, V, K, chunk, dt, &P) != KD_OK) return;
  check_cache_tiles(V, P.V_p, P.R_p);
  // block maxima: row n, blocks m0/32 .. +3 of V_p/32; collect loads: a
  // 16-byte load starting at v < V (v a multiple of 4) ends inside the row
  CHECK((P.V_p / kBlockRows) % 4 == 0 && P.V_p % 256 == 0, "block-maxima rows / logit rows");
  CHECK(((V - 1) / 4) * 4 + 4 <= P.V_p, "collect load past the row");
  const size_t eb = (size_t)P.eb;
  const std::vector<Buf> bufs = {
      {"W pad", P.off_wp, (size_t)V * P.d_p * eb, P.pad_d},
      {"H pad", P.off_hp, (size_t)P.R_p * P.d_p * eb, P.pad_d},
      {"block maxima", P.off_bmax, (size_t)P.R_p * (P.V_p / kBlockRows) * 4, true},
      {"theta", P.off_theta, (size_t)P.R_p * 4, true},
      {"counts", P.off_cnt, (size_t)P.R_p * 4, true},
      {"candidates", P.off_cand, (size_t)P.R_p * P.cap * 8, true},
      {"overflow", P.off_ovf, (size_t)P.R_p * 4, true},
      {"logits", P.off_z, (size_t)P.R_p * P.V_p * 4, true},
  };
  size_t prev_end = 0;
  for (const Buf& b : bufs) {
    if (!b.used) continue;
    CHECK(b.off % 256 == 0, "cache %s not 256-byte aligned", b.name);
    CHECK(b.off >= prev_end, "cache %s overlaps the previous buffer", b.name);
    CHECK(b.off + b.need <= P.total, "cache %s ends past the workspace", b.name);
    prev_end = b.off + b.need;
  }
  CHECK(P.cap >= 2 * K || P.cap == 8192, "candidate list shorter than 2K");
}

int main(int argc, char** argv) {
  for (int i = 1; i < argc; ++i)
    if (!strcmp(argv[i], "--plant") && i + 1 < argc) g_plant = argv[++i];

  check_acc_layout();
  check_hit_codes();
  check_grad_staging();
  check_cache_staging();

  // head-gradient RMW over ragged shapes, all three tile widths
  const int Vs[] = {1, 5, 127, 128, 255, 257, 3000, 5000, 201088};
  const int ds[] = {4, 64, 96, 128, 192, 320, 576, 704, 1900, 2880, 3072};
  for (int V : Vs)
    for (int d : ds) {
      check_accum(V, d, 128, false, 96 * 1024 / 8);
      check_accum(V, d, 192, false, 112 * 1024 / 8);
      if (d % 4 == 0) check_accum(V, d, 320, true, 144 * 1024 / 8);
    }

  // plans over ragged shapes, every mode, both dtypes
  const int64_t Ts[] = {1, 37, 700, 9500, 262144};
  const int64_t dps[] = {5, 64, 70, 576, 2880, 3072};
  const int64_t Vps[] = {11, 300, 3000, 128256, 201088, 2096896};
  const int64_t Ks[] = {1, 100, 4096};
  const int64_t chunks[] = {1, 37, 1000, 2048, 4096, 16384};
  for (int64_t T : Ts)
    for (int64_t d : dps)
      for (int64_t V : Vps)
        for (int64_t K : Ks)
          for (int64_t c : chunks)
            for (int dt = 0; dt < 2; ++dt)
              for (int mode = 0; mode < 3; ++mode) {
                check_plan(T, d, V, K, c, dt, mode, false);
                if (mode == kFused) check_plan(T, d, V, K, c, dt, mode, true);
              }

  // cache-builder plans over ragged shapes, both dtypes
  for (int64_t T : Ts)
    for (int64_t d : dps)
      for (int64_t V : Vps)
        for (int64_t K : Ks)
          for (int64_t c : chunks)
            for (int dt = 0; dt < 2; ++dt) check_cache_plan(T, d, V, K, c, dt);

  printf("index checks: %ld, failures: %ld%s%s\n", g_checks, g_fail, g_plant.empty() ? "" : ", planted: ",
         g_plant.c_str());
  return g_fail ? 1 : 0;
}
