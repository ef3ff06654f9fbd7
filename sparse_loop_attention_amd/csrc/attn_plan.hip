// Workspace planning and dispatch of an attend call to the per-row path or the
// tiled MFMA path.
//
// The tiled bf16 MFMA path serves bf16 stores with at least kMfmaMinRows
// active rows (prefill loops); the per-row path serves float32 stores and
// calls with few rows per head (decode), where a 32-row MFMA tile would idle.
#include <algorithm>

#include "fl_launch.hpp"

namespace fl {

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
    p.off_part = off;
    if (p.col_chunks > 1) off = align256(off + static_cast<uint64_t>(p.col_chunks) * sh * kpad * 4);
    p.off_logit = off;
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
