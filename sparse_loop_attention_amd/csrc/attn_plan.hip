// Workspace planning and dispatch of an attend call to the per-row path or the
// tiled MFMA path.
#include "fl_launch.hpp"

namespace fl {

hipError_t launch_rows(const fl_attend_args& x, const KvView& kv, const AttendPlan& p, hipStream_t st);

static uint64_t align256(uint64_t x) { return (x + 255) & ~uint64_t(255); }

AttendPlan plan_attend(const fl_attend_args& a) {
  AttendPlan p{};
  const fl_kv_desc& d = *a.kv;
  const bool lazy = a.mode == FL_ATTEND_LAZY;
  p.mfma = false;
  p.rows = a.n_active;
  p.keys = lazy ? a.n_keys : d.n_tokens;
  p.splits = static_cast<int>((p.keys + 63) / 64);
  const uint64_t sh = static_cast<uint64_t>(d.n_seq) * d.n_heads;
  const uint64_t rows = static_cast<uint64_t>(p.rows);
  uint64_t off = 0;
  p.off_part = off;
  off = align256(off + sh * rows * p.splits * (4 + 2 * static_cast<uint64_t>(d.head_dim)) * 4);
  p.off_logit = off;
  off = align256(off + 2 * sh * rows * static_cast<uint64_t>(p.keys) * 4);
  p.off_stat = off;
  off = align256(off + sh * rows * 16);
  p.off_gather = off;
  p.off_total = off;
  return p;
}

hipError_t launch_attend(const fl_attend_args& a, const KvView& kv, const AttendPlan& p, hipStream_t st) {
  return launch_rows(a, kv, p, st);
}

}  // namespace fl
