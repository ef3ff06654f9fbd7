// Workspace planning and dispatch of an attend call to the per-row path or the
// tiled MFMA path.
//
// The tiled bf16 MFMA path serves bf16 stores with at least kMfmaMinRows
// active rows (prefill loops); the per-row path serves float32 stores and
// calls with few rows per head (decode), where a 32-row MFMA tile would idle.
#include <algorithm>
#include <cstdlib>
#include <functional>
#include <map>
#include <mutex>
#include <queue>
#include <vector>

#include "fl_launch.hpp"

namespace fl {

// Forward pass of a full loop (MFMA path): 256-row tiles, 64-key tiles, one
// 8-wave workgroup per CU; MI355X has 8 XCDs of 32 CUs, and workgroup b of a
// launch starts on XCD b % 8.
constexpr int kFwdRows = 256, kFwdKeyTile = 64, kXcds = 8, kCusPerXcd = 32;

static int64_t fwd_key_tiles(int64_t n_rows, int64_t t) {
  return (std::min<int64_t>(n_rows, kFwdRows * (t + 1)) + kFwdKeyTile - 1) / kFwdKeyTile;
}

int fwd_split_items(int64_t n_rows, int u) {
  const int64_t T = (n_rows + kFwdRows - 1) / kFwdRows;
  int64_t n = 0;
  for (int64_t t = 0; t < T; ++t) n += u > 0 ? (fwd_key_tiles(n_rows, t) + u - 1) / u : 1;
  return static_cast<int>(n);
}

// Time, in key tiles, until the last forward workgroup ends, with the
// workgroups started in launch order (the order k_mfma_fwd maps them in: row
// tiles heaviest first, the parts of a split tile one after another, heads
// xcd + 8g on XCD xcd), each XCD starting its next workgroup on the first CU
// that frees.  A workgroup costs its key tiles plus a fixed overhead, one
// tile more for a part (its partial result is written and merged).
static double fwd_makespan(int64_t n_sh, int64_t n_rows, int u) {
  const int64_t T = (n_rows + kFwdRows - 1) / kFwdRows;
  std::vector<double> work;
  for (int64_t t = T - 1; t >= 0; --t) {
    const int64_t kt = fwd_key_tiles(n_rows, t);
    const int64_t p = u > 0 ? (kt + u - 1) / u : 1;
    for (int64_t j = 0; j < p; ++j) {
      const int64_t tiles = (j + 1) * kt / p - j * kt / p;
      work.push_back(static_cast<double>(tiles) + 2.0 + (p > 1 ? 1.0 : 0.0));
    }
  }
  const int64_t n_items = static_cast<int64_t>(work.size());
  const int64_t groups = (n_sh + kXcds - 1) / kXcds;
  double end = 0.0;
  for (int x = 0; x < kXcds; ++x) {
    std::priority_queue<double, std::vector<double>, std::greater<double>> cu;
    for (int c = 0; c < kCusPerXcd; ++c) cu.push(0.0);
    for (int64_t local = 0; local < groups * n_items; ++local) {
      const int64_t sh = x + kXcds * (local / n_items);
      if (sh >= n_sh) continue;
      const double t0 = cu.top();
      cu.pop();
      const double t1 = t0 + work[local % n_items];
      cu.push(t1);
      end = std::max(end, t1);
    }
  }
  return end;
}

int plan_fwd_split(int64_t n_sh, int64_t n_rows) {
  const int64_t T = (n_rows + kFwdRows - 1) / kFwdRows;
  // Only grids that leave CUs idle are split (parts of one head stay on one
  // XCD: n_sh >= 8).  From one workgroup per CU up, the split measured no
  // faster or slower: the chip's shared throughput, not the heaviest row
  // tile, then sets the time (16 heads x 4096 rows: 130 -> 133 us; 32 x 2048:
  // 74 -> 105 us), while 8 x 4096 went 124 -> 84 us.
  if (n_sh < kXcds || T < 2 || n_sh * T >= kXcds * kCusPerXcd) return 0;
  static std::mutex mu;
  static std::map<std::pair<int64_t, int64_t>, int> memo;
  std::lock_guard<std::mutex> lock(mu);
  const auto key = std::make_pair(n_sh, n_rows);
  const auto it = memo.find(key);
  if (it != memo.end()) return it->second;
  if (memo.size() >= 4096) memo.clear();                // shapes seen by a long-running caller
  const int64_t kt_max = fwd_key_tiles(n_rows, T - 1);
  int best = 0;
  double best_t = fwd_makespan(n_sh, n_rows, 0);
  for (int k = 2; k <= 8; ++k) {
    const int u = static_cast<int>((kt_max + k - 1) / k);
    if (u < 8) break;                                    // parts of at least 512 keys
    const double t = fwd_makespan(n_sh, n_rows, u);
    if (t < 0.9 * best_t) { best_t = t; best = u; }
  }
  memo[key] = best;
  return best;
}

int plan_fwd_pair(int64_t n_sh, int64_t n_rows) {
  const int64_t halves = (n_rows + 127) / 128, per = (halves + 1) / 2;
  if (halves < 2 || n_sh * per > kXcds * kCusPerXcd) return 0;
  return static_cast<int>(per);
}

// 256-row workgroups with 64-key tiles for lazy loops that fill the chip,
// else 128-row workgroups (64-key tiles up to head_dim 96, 32-key tiles at
// 128, whose four staged K and V chunks per thread would not fit the
// registers), or 64-row ones with 32-key tiles for grids too small even for
// those (more, lighter workgroups).
int plan_lazy_cfg(int64_t n_sh, int64_t n_rows) {
  const int64_t wg256 = n_sh * ((n_rows + 255) / 256);
  const int64_t wg128 = n_sh * ((n_rows + 127) / 128);
  return wg256 >= 512 ? 0 : wg128 >= 512 ? 1 : 2;
}

// The two passes of a lazy row tile as two workgroups: twice the workgroups
// (a finer balance over the CUs) and no pipeline restart between the passes;
// the two meet in the L2 of their XCD, which holds for >= 8 (sequence, head)
// rows (whole heads per XCD).  Measured (16 or 55 heads): it pays on grids of
// up to about 2.5 rounds of workgroups (32K workload, 2.4 / 1.2 / 0.64 rounds:
// 549 -> 532, 330 -> 318, 233 -> 203 us; the deep workload's loops of 1.2-1.4
// rounds 177 -> 159, 196 -> 182 us) and costs beyond (3.0-4.3 rounds:
// 352 -> 377, 480 -> 502 us: the output rows are read back from HBM by the
// second pass instead of from L2).  FLASHLOOP_LAZY_SPLIT=0 or =1 turns it off
// or on wherever it is possible.
static bool plan_lazy_split(int64_t n_sh, int64_t n_rows, int cfg) {
  if (n_sh < kXcds) return false;
  const char* e = getenv("FLASHLOOP_LAZY_SPLIT");
  if (e && e[0] == '0') return false;
  if (e && e[0] == '1') return true;
  const int64_t rows_per = lazy_cfg_rows(cfg);
  const int64_t wgs = n_sh * ((n_rows + rows_per - 1) / rows_per);
  const int64_t slots = (cfg == 0 ? 1 : cfg == 1 ? 2 : 4) * kXcds * kCusPerXcd;   // resident workgroups
  return 2 * wgs < 5 * slots;
}

hipError_t launch_rows(const fl_attend_args& x, const KvView& kv, const AttendPlan& p, hipStream_t st);
hipError_t launch_mfma(const fl_attend_args& x, const KvView& kv, const AttendPlan& p, hipStream_t st);

constexpr int kMfmaMinRows = 64;

static uint64_t align256(uint64_t x) { return (x + 255) & ~uint64_t(255); }

AttendPlan plan_attend(const fl_attend_args& a) {
  AttendPlan p{};
  const fl_kv_desc& d = *a.kv;
  const bool lazy = a.mode == FL_ATTEND_LAZY;
  const uint64_t sh = static_cast<uint64_t>(d.n_seq) * d.n_heads;
  const uint64_t D = static_cast<uint64_t>(d.head_dim);
  p.rows = a.n_active;
  p.keys = lazy ? a.n_keys : d.n_tokens;
  p.mfma = d.base_dtype == FL_BF16 && a.n_active >= kMfmaMinRows;
  const uint64_t rows = static_cast<uint64_t>(p.rows);
  uint64_t off = 0;
  if (p.mfma) {
    const uint64_t kpad = (static_cast<uint64_t>(p.keys) + 255) / 256 * 256;
    p.splits = 0;
    p.off_stat = off;
    off = align256(off + sh * rows * 16);
    p.off_gather = off;
    off = align256(off + (lazy ? 4 : 2) * sh * kpad * D * 2 + sh * kpad * 4);
    // enough column-mass workgroups to fill the chip: split the rows when
    // the key blocks alone are few
    const uint64_t kblk_wgs = sh * (kpad / 256);
    const uint64_t row_tiles = (rows + 63) / 64;
    uint64_t chunks = kblk_wgs >= 1024 ? 1 : (1024 + kblk_wgs - 1) / kblk_wgs;
    chunks = std::max<uint64_t>(1, std::min(chunks, row_tiles));
    p.col_rows = static_cast<int>((row_tiles + chunks - 1) / chunks * 64);
    p.col_chunks = static_cast<int>((rows + p.col_rows - 1) / p.col_rows);
    if (p.col_chunks < 1) p.col_chunks = 1;
    // a full loop over every row (rows = tokens = key slots) on >= 8 heads
    // sizes the ranges of each key block to its own rows (block b: rows from
    // 256 b on), so no range is empty and the largest is small: the largest
    // range length (a multiple of 64) that still gives >= 512 items (two per
    // CU: 1024 and 2048 measured 1 % slower on 16 heads x 4096 rows)
    p.col_var_rows = 0;
    p.col_items = 0;
    if (!lazy && !a.active_idx && p.col_chunks > 1 && sh >= 8) {
      const uint64_t n_kblk = kpad / 256;
      auto items_for = [&](uint64_t r) {
        uint64_t n = 0;
        for (uint64_t b = 0; b < n_kblk; ++b) n += (rows - 256 * b + r - 1) / r;
        return n;
      };
      uint64_t r = 64 * row_tiles;
      while (r > 64 && sh * items_for(r) < 512) r -= 64;
      p.col_var_rows = static_cast<int>(r);
      p.col_items = static_cast<int>(items_for(r));
      p.col_chunks = static_cast<int>((rows + r - 1) / r);
      p.col_rows = static_cast<int>(r);
    }
    p.off_part = off;
    if (p.col_chunks > 1) off = align256(off + static_cast<uint64_t>(p.col_chunks) * sh * kpad * 4);
    // full loops: the ranges of one key block run on one XCD when there are
    // >= 8 heads, and the last one to finish adds the partial sums (one
    // counter per block).  Lazy loops keep the reduction launch: the fused
    // ending cost the two-pass kernel more registers than the launch saves.
    p.col_fused = !lazy && p.col_chunks > 1 && sh >= 8;
    p.off_ccount = off;                                  // counters, then as many XCD masks
    if (p.col_fused) off = align256(off + 2 * sh * (kpad / 256) * 4);
    p.off_logit = off;
    // forward key split of full loops: one partial (acc, max, sum of every
    // lane of the 512-thread workgroup) per workgroup, one counter per row tile
    p.fsplit_u = lazy ? 0 : plan_fwd_split(static_cast<int64_t>(sh), p.rows);
    p.f_tiles = static_cast<int>((rows + 255) / 256);
    p.f_items = p.fsplit_u > 0 ? fwd_split_items(p.rows, p.fsplit_u) : p.f_tiles;
    p.fpair = lazy || p.fsplit_u > 0 ? 0 : plan_fwd_pair(static_cast<int64_t>(sh), p.rows);
    p.lazy_cfg = lazy ? plan_lazy_cfg(static_cast<int64_t>(sh), p.rows) : 0;
    p.lsplit = lazy && plan_lazy_split(static_cast<int64_t>(sh), p.rows, p.lazy_cfg);
    p.off_fpart = off;
    p.off_fcount = off;
    p.off_lmass = off;
    if (p.lsplit) {
      // one partial (acc, max, sum of every lane) per row tile, written by the
      // current-loop pass when it ends before the previous-loop pass
      const uint64_t rows_per = lazy_cfg_rows(p.lazy_cfg), nt = 2 * rows_per;
      p.f_tiles = static_cast<int>((rows + rows_per - 1) / rows_per);
      off = align256(off + sh * p.f_tiles * (D / 8 + 1) * nt * 16);
      p.off_fcount = off;                                // counters, then as many XCD masks
      off = align256(off + 2 * sh * p.f_tiles * 4);
      p.off_lmass = off;
      off = align256(off + sh * rows * 4);
    } else if (p.fsplit_u > 0) {
      off = align256(off + sh * p.f_items * (D / 8 + 1) * 512 * 16);   // D/8 float4 of acc + (max, sum)
      p.off_fcount = off;                                // counters, then as many XCD masks
      off = align256(off + 2 * sh * p.f_tiles * 4);
    }
    p.off_pcol = off;
    if (lazy) {
      const uint64_t rows_per = lazy_cfg_rows(p.lazy_cfg);
      off = align256(off + sh * ((rows + rows_per - 1) / rows_per) * kpad * 4);
    }
    p.off_total = off;
    return p;
  }
  p.splits = 0;
  p.off_part = off;
  p.off_logit = off;                                     // per-row path: logits of every row for the column pass
  off = align256(off + 2 * sh * rows * static_cast<uint64_t>(p.keys) * 4);
  p.off_stat = off;
  off = align256(off + sh * rows * 16);
  p.off_gather = off;
  p.off_total = off;
  return p;
}

hipError_t launch_attend(const fl_attend_args& a, const KvView& kv, const AttendPlan& p, hipStream_t st) {
  return p.mfma ? launch_mfma(a, kv, p, st) : launch_rows(a, kv, p, st);
}

}  // namespace fl
